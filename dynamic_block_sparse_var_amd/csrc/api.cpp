// api.cpp -- the extern "C" entry points of libprism: host-side validation (no HIP call
// happens before an argument check has passed), error strings, and dispatch to the stage
// launchers in the .hip sources.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "prism_internal.h"

namespace prism {

const ShapeEntry kShapes[16] = {PRISM_SHAPES};

static thread_local char g_err[512];

prism_status fail(prism_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

prism_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PRISM_OK;
  return fail(PRISM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

prism_status check_launch(const char* what) { return check_hip(hipGetLastError(), what); }

namespace {
struct TraceSlot {
  char name[32];
  hipEvent_t start, stop;
};
TraceSlot g_trace[8];
int g_trace_n = 0;
}  // namespace

KernelTrace::KernelTrace(const char* kernel, hipStream_t st) : st_(st) {
  for (int i = 0; i < g_trace_n; ++i)
    if (strcmp(g_trace[i].name, kernel) == 0) {
      (void)hipEventRecord(g_trace[i].start, st);
      stop_ = g_trace[i].stop;
      return;
    }
}

KernelTrace::~KernelTrace() {
  if (stop_) (void)hipEventRecord(stop_, st_);
}

prism_status need_ptr(const void* p, const char* name) {
  return p ? PRISM_OK : fail(PRISM_E_NULL, "%s is NULL", name);
}

prism_status need_aligned(const void* p, const char* name) {
  if (!p) return fail(PRISM_E_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15u) return fail(PRISM_E_ALIGN, "%s is not 16-byte aligned", name);
  return PRISM_OK;
}

prism_status validate_problem(const prism_problem* pb) {
  if (!pb) return fail(PRISM_E_NULL, "problem is NULL");
  if (pb->T <= 0 || pb->H <= 0 || pb->W <= 0 || pb->T % kZone || pb->H % kZone || pb->W % kZone)
    return fail(PRISM_E_SHAPE, "grid %dx%dx%d: each axis must be a positive multiple of 8", pb->T, pb->H,
                pb->W);
  int64_t Z = (int64_t)(pb->T / kZone) * (pb->H / kZone) * (pb->W / kZone);
  if (Z > kMaxZones) return fail(PRISM_E_SHAPE, "%lld zones exceed the limit of %d", (long long)Z, kMaxZones);
  if (pb->heads <= 0 || pb->heads > 256) return fail(PRISM_E_SHAPE, "heads = %d not in [1, 256]", pb->heads);
  if (pb->head_dim != 64 && pb->head_dim != 128)
    return fail(PRISM_E_SHAPE, "head_dim = %d not in {64, 128}", pb->head_dim);
  if (pb->groups <= 0 || pb->heads % pb->groups)
    return fail(PRISM_E_SHAPE, "groups = %d must divide heads = %d", pb->groups, pb->heads);
  if (pb->dtype != PRISM_F32 && pb->dtype != PRISM_BF16) return fail(PRISM_E_DTYPE, "dtype = %d", pb->dtype);
  int64_t elems = Z * kZoneVol * (int64_t)pb->heads * pb->head_dim;
  if (elems >= (int64_t(1) << 31)) return fail(PRISM_E_SHAPE, "tensor of %lld elements too large", (long long)elems);
  return PRISM_OK;
}

Geom make_geom(const prism_problem* pb) {
  Geom g;
  g.T = pb->T; g.H = pb->H; g.W = pb->W;
  g.ZT = pb->T / kZone; g.ZH = pb->H / kZone; g.ZW = pb->W / kZone;
  g.Z = g.ZT * g.ZH * g.ZW;
  g.heads = pb->heads; g.d = pb->head_dim; g.groups = pb->groups; g.hpg = pb->heads / pb->groups;
  g.nbmax = 8 * g.Z;
  g.N = (int64_t)pb->T * pb->H * pb->W;
  g.bf16 = pb->dtype == PRISM_BF16;
  g.esize = g.bf16 ? 2 : 4;
  return g;
}

}  // namespace prism

using namespace prism;

#define PRISM_TRY(x)                       \
  do {                                     \
    prism_status _s = (x);                 \
    if (_s != PRISM_OK) return _s;         \
  } while (0)

extern "C" {

int32_t prism_abi_version(void) { return PRISM_ABI_VERSION; }

const char* prism_status_string(prism_status s) {
  switch (s) {
    case PRISM_OK: return "ok";
    case PRISM_E_NULL: return "null pointer";
    case PRISM_E_SHAPE: return "unsupported shape";
    case PRISM_E_RANGE: return "argument out of range";
    case PRISM_E_DTYPE: return "unknown dtype";
    case PRISM_E_ALIGN: return "misaligned pointer";
    case PRISM_E_WORKSPACE: return "workspace too small";
    case PRISM_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* prism_last_error(void) { return g_err; }

prism_status prism_trace_kernel(const char* kernel, void* start_event, void* stop_event) {
  g_err[0] = 0;
  if (!kernel) {
    g_trace_n = 0;
    return PRISM_OK;
  }
  if (!start_event || !stop_event) return fail(PRISM_E_NULL, "trace events are NULL");
  if (strlen(kernel) >= sizeof(g_trace[0].name)) return fail(PRISM_E_RANGE, "kernel name too long");
  int slot = -1;
  for (int i = 0; i < g_trace_n; ++i)
    if (strcmp(g_trace[i].name, kernel) == 0) slot = i;
  if (slot < 0) {
    if (g_trace_n >= 8) return fail(PRISM_E_RANGE, "all 8 trace slots in use");
    slot = g_trace_n++;
    strcpy(g_trace[slot].name, kernel);
  }
  g_trace[slot].start = static_cast<hipEvent_t>(start_event);
  g_trace[slot].stop = static_cast<hipEvent_t>(stop_event);
  return PRISM_OK;
}

prism_status prism_set_launch_order(int32_t heavy_first) {
  g_err[0] = 0;
  if (heavy_first != 0 && heavy_first != 1) return fail(PRISM_E_RANGE, "heavy_first = %d must be 0 or 1", heavy_first);
  set_heavy_first_order(heavy_first == 1);
  return PRISM_OK;
}

int32_t prism_shape_table(int32_t* edges) {
  if (!edges) return 0;
  for (int i = 0; i < 16; ++i) {
    edges[3 * i + 0] = kShapes[i].bT;
    edges[3 * i + 1] = kShapes[i].bH;
    edges[3 * i + 2] = kShapes[i].bW;
  }
  return 16;
}

prism_status prism_audio_norms(const prism_problem* pb, const void* hhat, int32_t channels, int32_t squared, float* a,
                               void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(hhat, "hhat"));
  PRISM_TRY(need_aligned(a, "a"));
  if (channels <= 0 || channels % 8 != 0 || channels > (1 << 20))
    return fail(PRISM_E_RANGE, "channels = %d must be a positive multiple of 8, at most 2^20", channels);
  if (squared != 0 && squared != 1) return fail(PRISM_E_RANGE, "squared = %d must be 0 or 1", squared);
  Geom gm = make_geom(pb);
  return launch_audio_norms(gm, hhat, channels, squared, a, (hipStream_t)stream);
}

prism_status prism_zone_stats(const prism_problem* pb, const void* v, const float* a, float eps, float* g,
                              float* rho, float* zone_audio, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(g, "g"));
  PRISM_TRY(need_aligned(rho, "rho"));
  if (a) {
    PRISM_TRY(need_aligned(a, "a"));
    PRISM_TRY(need_aligned(zone_audio, "zone_audio"));
  }
  if (!(eps > 0.f) || !isfinite(eps)) return fail(PRISM_E_RANGE, "eps = %g must be finite and > 0", (double)eps);
  Geom gm = make_geom(pb);
  return launch_zone_stats(gm, v, a, eps, g, rho, zone_audio, (hipStream_t)stream);
}

prism_status prism_assign_shapes(const prism_problem* pb, const float* g, const float* rho, float tau128,
                                 float tau256, uint8_t* shape_idx, int32_t* zone_block_off, int32_t* block_start,
                                 void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(g, "g"));
  PRISM_TRY(need_aligned(rho, "rho"));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  PRISM_TRY(need_aligned(zone_block_off, "zone_block_off"));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  if (!isfinite(tau128) || !isfinite(tau256) || tau256 < 0.f || tau128 < tau256)
    return fail(PRISM_E_RANGE, "thresholds tau128 = %g, tau256 = %g must satisfy 0 <= tau256 <= tau128",
                (double)tau128, (double)tau256);
  Geom gm = make_geom(pb);
  return launch_assign_shapes(gm, g, rho, tau128, tau256, shape_idx, zone_block_off, block_start,
                              (hipStream_t)stream);
}

prism_status prism_fixed_shapes(const prism_problem* pb, int32_t shape_index, uint8_t* shape_idx,
                                int32_t* zone_block_off, int32_t* block_start, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  PRISM_TRY(need_aligned(zone_block_off, "zone_block_off"));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  if (shape_index < 0 || shape_index > 15) return fail(PRISM_E_RANGE, "shape_index = %d not in [0, 15]", shape_index);
  Geom gm = make_geom(pb);
  return launch_fixed_shapes(gm, shape_index, shape_idx, zone_block_off, block_start, (hipStream_t)stream);
}

prism_status prism_permute(const prism_problem* pb, const uint8_t* shape_idx, int32_t inverse, int32_t count,
                           const void* const* src, void* const* dst, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  if (inverse != 0 && inverse != 1) return fail(PRISM_E_RANGE, "inverse = %d must be 0 or 1", inverse);
  if (count < 1 || count > 4) return fail(PRISM_E_RANGE, "count = %d not in [1, 4]", count);
  PRISM_TRY(need_ptr(src, "src"));
  PRISM_TRY(need_ptr(dst, "dst"));
  for (int i = 0; i < count; ++i) {
    PRISM_TRY(need_aligned(src[i], "src[i]"));
    PRISM_TRY(need_aligned(dst[i], "dst[i]"));
  }
  Geom gm = make_geom(pb);
  return launch_permute(gm, shape_idx, inverse, count, src, dst, (hipStream_t)stream);
}

prism_status prism_permute_pool(const prism_problem* pb, const uint8_t* shape_idx, const int32_t* zone_block_off,
                                int32_t count, const void* const* src, void* const* dst, float* const* xbar,
                                void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  PRISM_TRY(need_aligned(zone_block_off, "zone_block_off"));
  if (count < 1 || count > 4) return fail(PRISM_E_RANGE, "count = %d not in [1, 4]", count);
  PRISM_TRY(need_ptr(src, "src"));
  PRISM_TRY(need_ptr(dst, "dst"));
  for (int i = 0; i < count; ++i) {
    PRISM_TRY(need_aligned(src[i], "src[i]"));
    PRISM_TRY(need_aligned(dst[i], "dst[i]"));
    if (xbar && xbar[i]) PRISM_TRY(need_aligned(xbar[i], "xbar[i]"));
  }
  Geom gm = make_geom(pb);
  return launch_permute_pool(gm, shape_idx, zone_block_off, count, src, dst, xbar, (hipStream_t)stream);
}

prism_status prism_pool_blocks(const prism_problem* pb, const int32_t* block_start, int32_t count,
                               const void* const* x_perm, float* const* xbar, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  if (count < 1 || count > 4) return fail(PRISM_E_RANGE, "count = %d not in [1, 4]", count);
  PRISM_TRY(need_ptr(x_perm, "x_perm"));
  PRISM_TRY(need_ptr(xbar, "xbar"));
  for (int i = 0; i < count; ++i) {
    PRISM_TRY(need_aligned(x_perm[i], "x_perm[i]"));
    PRISM_TRY(need_aligned(xbar[i], "xbar[i]"));
  }
  Geom gm = make_geom(pb);
  return launch_pool(gm, block_start, count, x_perm, xbar, (hipStream_t)stream);
}

prism_status prism_select_blocks(const prism_problem* pb, const int32_t* block_start, const float* qbar,
                                 const float* kbar, float sm_scale, int32_t k_abs, double k_frac, double p,
                                 int32_t* sel_count, int32_t* sel_idx, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(qbar, "qbar"));
  PRISM_TRY(need_aligned(kbar, "kbar"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  if (k_abs < 0) return fail(PRISM_E_RANGE, "k_abs = %d must be >= 0", k_abs);
  if (!(k_frac >= 0.0 && k_frac <= 1.0)) return fail(PRISM_E_RANGE, "k_frac = %g not in [0, 1]", k_frac);
  if (!(p >= 0.0 && p <= 1.0)) return fail(PRISM_E_RANGE, "p = %g not in [0, 1]", p);
  Geom gm = make_geom(pb);
  return launch_select(gm, block_start, qbar, kbar, sm_scale, k_abs, k_frac, p, sel_count, sel_idx,
                       (hipStream_t)stream);
}

size_t prism_bsa_fwd_workspace_bytes(const prism_problem* pb) {
  if (validate_problem(pb) != PRISM_OK) return 0;
  Geom gm = make_geom(pb);
  return bsa_fwd_workspace_bytes(gm);
}

// the optional forward workspace: NULL, or aligned and large enough
static prism_status check_fwd_workspace(const Geom& gm, const void* workspace, size_t workspace_bytes) {
  if (!workspace) return PRISM_OK;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(PRISM_E_ALIGN, "workspace not 256-byte aligned");
  const size_t need = bsa_fwd_workspace_bytes(gm);
  if (workspace_bytes < need)
    return fail(PRISM_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return PRISM_OK;
}

prism_status prism_bsa_fwd(const prism_problem* pb, const int32_t* block_start, const int32_t* sel_count,
                           const int32_t* sel_idx, float sm_scale, const void* q, const void* k, const void* v,
                           void* o, void* o_lo, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  PRISM_TRY(need_aligned(q, "q"));
  PRISM_TRY(need_aligned(k, "k"));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(o, "o"));
  if (o_lo) PRISM_TRY(need_aligned(o_lo, "o_lo"));
  PRISM_TRY(need_aligned(lse, "lse"));
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  Geom gm = make_geom(pb);
  PRISM_TRY(check_fwd_workspace(gm, workspace, workspace_bytes));
  return launch_bsa_fwd(gm, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, gm.bf16 ? o_lo : nullptr, lse,
                        workspace, block_rows(), (hipStream_t)stream);
}

size_t prism_bsa_bwd_workspace_bytes(const prism_problem* pb) {
  if (validate_problem(pb) != PRISM_OK) return 0;
  Geom gm = make_geom(pb);
  return bsa_bwd_workspace_bytes(gm);
}

prism_status prism_bsa_bwd(const prism_problem* pb, const int32_t* block_start, const int32_t* sel_count,
                           const int32_t* sel_idx, float sm_scale, const void* q, const void* k, const void* v,
                           const void* o, const void* o_lo, const void* dout, const float* lse, float* dq, float* dk,
                           float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  PRISM_TRY(need_aligned(q, "q"));
  PRISM_TRY(need_aligned(k, "k"));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(o, "o"));
  if (o_lo) PRISM_TRY(need_aligned(o_lo, "o_lo"));
  PRISM_TRY(need_aligned(dout, "dout"));
  PRISM_TRY(need_aligned(lse, "lse"));
  PRISM_TRY(need_aligned(dq, "dq"));
  PRISM_TRY(need_aligned(dk, "dk"));
  PRISM_TRY(need_aligned(dv, "dv"));
  PRISM_TRY(need_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(PRISM_E_ALIGN, "workspace not 256-byte aligned");
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  Geom gm = make_geom(pb);
  size_t need = bsa_bwd_workspace_bytes(gm);
  if (workspace_bytes < need)
    return fail(PRISM_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return launch_bsa_bwd(gm, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, gm.bf16 ? o_lo : nullptr, dout,
                        lse, dq, dk, dv, workspace, block_rows(), block_rows(), (hipStream_t)stream);
}

prism_status prism_bsa_bwd_noalloc(const prism_problem* pb, const int32_t* block_start, const int32_t* sel_count,
                                   const int32_t* sel_idx, float sm_scale, const void* q, const void* k,
                                   const void* v, const void* o, const void* o_lo, const void* dout,
                                   const float* lse, float* dq, float* dk, float* dv, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  PRISM_TRY(need_aligned(q, "q"));
  PRISM_TRY(need_aligned(k, "k"));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(o, "o"));
  if (o_lo) PRISM_TRY(need_aligned(o_lo, "o_lo"));
  PRISM_TRY(need_aligned(dout, "dout"));
  PRISM_TRY(need_aligned(lse, "lse"));
  PRISM_TRY(need_aligned(dq, "dq"));
  PRISM_TRY(need_aligned(dk, "dk"));
  PRISM_TRY(need_aligned(dv, "dv"));
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  Geom gm = make_geom(pb);
  const size_t need = bsa_bwd_workspace_bytes(gm);
  if (need > kNoAllocScratchBytes)
    return fail(PRISM_E_WORKSPACE, "backward needs %zu bytes of scratch, the allocation-free entry point has %zu",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  PRISM_TRY(noalloc_scratch(&ws));
  return launch_bsa_bwd(gm, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, gm.bf16 ? o_lo : nullptr, dout,
                        lse, dq, dk, dv, ws, block_rows(), block_rows(), (hipStream_t)stream);
}

size_t prism_bsa_bwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

// ---- token-order interface of the attention ---------------------------------------------

prism_status prism_bsa_fwd_tok(const prism_problem* pb, const uint8_t* shape_idx, const int32_t* block_start,
                               const int32_t* sel_count, const int32_t* sel_idx, float sm_scale, const void* q,
                               const void* k, const void* v, void* o, void* o_lo, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  PRISM_TRY(need_aligned(q, "q"));
  PRISM_TRY(need_aligned(k, "k"));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(o, "o"));
  if (o_lo) PRISM_TRY(need_aligned(o_lo, "o_lo"));
  PRISM_TRY(need_aligned(lse, "lse"));
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  Geom gm = make_geom(pb);
  PRISM_TRY(check_fwd_workspace(gm, workspace, workspace_bytes));
  return launch_bsa_fwd(gm, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, gm.bf16 ? o_lo : nullptr, lse,
                        workspace, token_rows(gm, shape_idx), (hipStream_t)stream);
}

// the block-order backward workspace, then a block-order copy of dO
static size_t dout_copy_offset(const Geom& gm) { return (bsa_bwd_workspace_bytes(gm) + 255) & ~(size_t)255; }

size_t prism_bsa_bwd_tok_workspace_bytes(const prism_problem* pb) {
  if (validate_problem(pb) != PRISM_OK) return 0;
  Geom gm = make_geom(pb);
  return dout_copy_offset(gm) + (size_t)gm.heads * (size_t)gm.N * (size_t)gm.d * (size_t)gm.esize;
}

prism_status prism_bsa_bwd_tok(const prism_problem* pb, const uint8_t* shape_idx, const int32_t* block_start,
                               const int32_t* sel_count, const int32_t* sel_idx, float sm_scale, const void* q,
                               const void* k, const void* v, const void* o, const void* o_lo, const void* dout,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  PRISM_TRY(validate_problem(pb));
  PRISM_TRY(need_aligned(shape_idx, "shape_idx"));
  PRISM_TRY(need_aligned(block_start, "block_start"));
  PRISM_TRY(need_aligned(sel_count, "sel_count"));
  PRISM_TRY(need_aligned(sel_idx, "sel_idx"));
  PRISM_TRY(need_aligned(q, "q"));
  PRISM_TRY(need_aligned(k, "k"));
  PRISM_TRY(need_aligned(v, "v"));
  PRISM_TRY(need_aligned(o, "o"));
  if (o_lo) PRISM_TRY(need_aligned(o_lo, "o_lo"));
  PRISM_TRY(need_aligned(dout, "dout"));
  PRISM_TRY(need_aligned(lse, "lse"));
  PRISM_TRY(need_aligned(dq, "dq"));
  PRISM_TRY(need_aligned(dk, "dk"));
  PRISM_TRY(need_aligned(dv, "dv"));
  PRISM_TRY(need_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(PRISM_E_ALIGN, "workspace not 256-byte aligned");
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(PRISM_E_RANGE, "sm_scale = %g must be finite and > 0", (double)sm_scale);
  Geom gm = make_geom(pb);
  const size_t need = prism_bsa_bwd_tok_workspace_bytes(pb);
  if (workspace_bytes < need)
    return fail(PRISM_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  void* dout_p = static_cast<uint8_t*>(workspace) + dout_copy_offset(gm);
  const void* src[1] = {dout};
  void* dst[1] = {dout_p};
  PRISM_TRY(launch_permute(gm, shape_idx, 0, 1, src, dst, (hipStream_t)stream));
  const RowMap tok = token_rows(gm, shape_idx);
  return launch_bsa_bwd(gm, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, gm.bf16 ? o_lo : nullptr, dout_p,
                        lse, dq, dk, dv, workspace, tok, tok, (hipStream_t)stream);
}

}  // extern "C"
