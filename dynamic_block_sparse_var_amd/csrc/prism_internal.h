// prism_internal.h -- definitions shared by the HIP sources of libprism (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prism.h"
#include "index_math.h"

namespace prism {

constexpr int kZone = 8;      // macro-zone edge (RG KI)
constexpr int kZoneVol = 512; // tokens per zone
constexpr int kMaxZones = 2048;  // 8 * Z blocks must fit one selection workgroup (64 entries per thread)

// Geometry derived from a validated prism_problem.
struct Geom {
  int T, H, W, ZT, ZH, ZW, Z, heads, d, groups, hpg, nbmax;
  int64_t N;
  int esize;  // bytes per element
  bool bf16;
};

Geom make_geom(const prism_problem* pb);

// Error plumbing (host).
prism_status fail(prism_status s, const char* fmt, ...);
prism_status check_hip(hipError_t e, const char* what);
prism_status check_launch(const char* what);

// Measurement hook (prism_trace_kernel): records the caller's events around one launch of the
// named kernel if a hook is set for it.  Construct right before the launch.
class KernelTrace {
 public:
  KernelTrace(const char* kernel, hipStream_t st);
  ~KernelTrace();

 private:
  hipEvent_t stop_ = nullptr;
  hipStream_t st_;
};

// Host-side validation helpers (no HIP calls).
prism_status validate_problem(const prism_problem* pb);
prism_status need_ptr(const void* p, const char* name);
prism_status need_aligned(const void* p, const char* name);

// Candidate shapes (RG KI: 16 shapes; volumes {64,128,256}, RG M2).  Reading: power-of-two
// edges in {2,4,8}, which gives exactly 7 + 6 + 3 = 16 boxes.  Index order = volume ascending,
// then (bT,bH,bW) lexicographic.  Entries are (bT, bH, bW, volume).
#define PRISM_SHAPES                                                                        \
  {2, 4, 8, 64}, {2, 8, 4, 64}, {4, 2, 8, 64}, {4, 4, 4, 64}, {4, 8, 2, 64}, {8, 2, 4, 64}, \
  {8, 4, 2, 64}, {2, 8, 8, 128}, {4, 4, 8, 128}, {4, 8, 4, 128}, {8, 2, 8, 128},            \
  {8, 4, 4, 128}, {8, 8, 2, 128}, {4, 8, 8, 256}, {8, 4, 8, 256}, {8, 8, 4, 256}
struct ShapeEntry { int16_t bT, bH, bW, vol; };
extern const ShapeEntry kShapes[16];
// Device copy of the table, one per translation unit that uses it (constant memory).
#define PRISM_DEVICE_SHAPES static __constant__ ShapeEntry c_shapes[16] = {PRISM_SHAPES};

// ---- device helpers ------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Where the attention kernels put an output row: block order [heads, N, d] when shape_idx is
// NULL, else token order [N, heads, d] (the row's token from its zone's shape).
struct RowMap {
  const uint8_t* shape_idx;  // [groups, Z] or NULL
  int H, W, ZH, ZW, Z;
};
inline RowMap block_rows() { return RowMap{nullptr, 0, 0, 0, 0, 0}; }
inline RowMap token_rows(const Geom& g, const uint8_t* shape_idx) {
  return RowMap{shape_idx, g.H, g.W, g.ZH, g.ZW, g.Z};
}
// Row index (in rows of d elements) of block-order row `row` of head h (group grp); `shapes` is
// the translation unit's device copy of the shape table.
__device__ __forceinline__ int64_t out_row(const RowMap& rm, const ShapeEntry* shapes, int grp, int h, int heads,
                                           int64_t N, int row) {
  if (!rm.shape_idx) return (int64_t)h * N + row;
  const int m = row >> 9;
  const ShapeEntry se = shapes[rm.shape_idx[(int64_t)grp * rm.Z + m]];
  return zone_pos_token(m, row & 511, se.bT, se.bH, se.bW, rm.H, rm.W, rm.ZH, rm.ZW) * heads + h;
}

// ---- stage launchers (defined in the .hip files; arguments already validated) ---------

prism_status launch_audio_norms(const Geom& g, const void* hhat, int channels, int squared, float* a,
                                hipStream_t st);
prism_status launch_zone_stats(const Geom& g, const void* v, const float* a, float eps, float* gout,
                               float* rho, float* zone_audio, hipStream_t st);
prism_status launch_assign_shapes(const Geom& g, const float* gin, const float* rho, float tau128,
                                  float tau256, uint8_t* shape_idx, int32_t* zone_block_off,
                                  int32_t* block_start, hipStream_t st);
prism_status launch_fixed_shapes(const Geom& g, int shape_index, uint8_t* shape_idx, int32_t* zone_block_off,
                                 int32_t* block_start, hipStream_t st);
prism_status launch_permute(const Geom& g, const uint8_t* shape_idx, int inverse, int count,
                            const void* const* src, void* const* dst, hipStream_t st);
prism_status launch_pool(const Geom& g, const int32_t* block_start, int count,
                         const void* const* x, float* const* xbar, hipStream_t st);
prism_status launch_permute_pool(const Geom& g, const uint8_t* shape_idx, const int32_t* zone_block_off,
                                 int count, const void* const* src, void* const* dst, float* const* xbar,
                                 hipStream_t st);
prism_status launch_select(const Geom& g, const int32_t* block_start, const float* qbar,
                           const float* kbar, float sm_scale, int32_t k_abs, double k_frac,
                           double p, int32_t* sel_count, int32_t* sel_idx, hipStream_t st);
// out: where o, o_lo (forward) and dq, dk, dv (backward) go; o_in: where the backward reads o,
// o_lo.  dout and everything else stay in block order.
// ws: NULL or bsa_fwd_workspace_bytes(g) bytes of scratch (the launch order of the forward).
size_t bsa_fwd_workspace_bytes(const Geom& g);
void set_heavy_first_order(bool on);
prism_status launch_bsa_fwd(const Geom& g, const int32_t* block_start, const int32_t* sel_count,
                            const int32_t* sel_idx, float sm_scale, const void* q, const void* k,
                            const void* v, void* o, void* o_lo, float* lse, void* ws, const RowMap& out,
                            hipStream_t st);
size_t bsa_bwd_workspace_bytes(const Geom& g);
// The allocation-free backward (prism_bsa_bwd_noalloc): its workspace is a device array of
// kNoAllocScratchBytes per device; noalloc_scratch gives the current device's copy.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
prism_status noalloc_scratch(void** out);
prism_status launch_bsa_bwd(const Geom& g, const int32_t* block_start, const int32_t* sel_count,
                            const int32_t* sel_idx, float sm_scale, const void* q, const void* k,
                            const void* v, const void* o, const void* o_lo, const void* dout,
                            const float* lse, float* dq, float* dk, float* dv, void* ws,
                            const RowMap& o_in, const RowMap& out, hipStream_t st);

}  // namespace prism
