"""The kernels' index arithmetic on the CPU (no GPU): dynamic_block_sparse_var_amd/csrc/
index_math.h is compiled into tests/index_check.cpp with the host compiler under
AddressSanitizer + UndefinedBehaviorSanitizer and checked exhaustively:

* LDS tiles (head_dim 64 and 128): the direct-to-LDS staging writes every 16-byte slot of a
  64-row tile once, with the chunk that the reads expect there; every operand read and every
  transposing read addresses the intended element inside the tile; the swizzle spreads 16 rows
  at one chunk, and a half-wave's 4 rows x 4 chunks, over distinct slots;
* unit order: xcd_atom is a bijection for every unit count up to 4096; block_of_row finds the
  block of every row on random layouts of 64/128/256-row blocks;
* block order: zone_pos_token (the kernels' token of a block-order row) is the inverse of the
  oracle's block layout on a grid whose zones take every one of the 16 shapes, compared with
  oracle.block_layout, which enumerates the layout independently.

Also: the bounds-checked build (-DPRISM_DEBUG, kernels asserting that the rows, tiles and list
entries they touch lie inside their tensors) compiles for gfx950."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_block_sparse_var_amd", "csrc")
MAIN = os.path.join(ROOT, "tests", "index_check.cpp")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("idx") / "index_check")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", CSRC, MAIN, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "cannot find" in r.stderr and "san" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr
    return out


def _run(exe, *args, stdin=None):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, input=stdin, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    return r.stdout


def test_lds_tile_addressing(exe):
    out = _run(exe, "tiles")
    assert "tiles D=64 checked" in out and "tiles D=128 checked" in out


def test_unit_order_and_block_lookup(exe):
    assert "units checked" in _run(exe, "units")


def test_block_order_matches_oracle_layout(exe):
    T, H, W = 24, 32, 40                      # 3 x 4 x 5 = 60 zones
    Z = (T // 8) * (H // 8) * (W // 8)
    rng = np.random.default_rng(77)
    shape_idx = np.concatenate([np.arange(16), rng.integers(0, 16, Z - 16)]).astype(np.uint8)
    rng.shuffle(shape_idx)
    edges, _ = oracle.candidates()
    stdin = "\n".join(" ".join(str(int(e)) for e in row) for row in edges) + "\n"
    out = _run(exe, "layout", T, H, W, *shape_idx.tolist(), stdin=stdin)
    pos = np.array([int(x) for x in out.split()], np.int64)
    opos, _, _ = oracle.block_layout(T, H, W, shape_idx[None, :])
    assert pos.shape == (T * H * W,)
    np.testing.assert_array_equal(pos, opos[0])


def test_bounds_checked_build_compiles(tmp_path):
    from dynamic_block_sparse_var_amd import build as b

    out = b.build(extra=["-DPRISM_DEBUG"], out=str(tmp_path / "libprism_debug.so"))
    assert os.path.getsize(out) > 0
