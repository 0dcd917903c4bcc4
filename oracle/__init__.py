"""CPU oracle for the m=1 decode matvec path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The HIP library never imports, links or calls it, and it never calls
the HIP library: the two share no code.  Inputs come from ``synth`` (seeded generators only).

What it computes (docs.rs pages of memra-engine 0.125.0):

* RMSNorm, from the fused-producer gate page (src/bin/q8_fuse_gate.rs, module doc and
  ``run_shape``): per row z = x * w / sqrt(mean(x^2) + eps), eps = 1e-6 given as an f32.
  Here, in f64: ss = the exactly rounded sum of x_j^2 (``math.fsum``; each square is exact in
  f64), s = 1 / sqrt(ss / ncols + eps), z64_j = (x_j * w_j) * s (x_j * w_j is exact in f64).
  The f32 output the producer stores is z32 = float32(z64).
* q8_1 quantisation (same page: int8 qs plus one f32 scale per 32 values, ``id = 1/d``),
  in f32 -- see ``oracle.c``.
* The three GEMVs of the bench page (src/bin/gemv_e4m3_bench.rs, module doc THE COMPARISON
  and THE BLOCK-128 ARM), f64 terms and sums -- see ``oracle.c``.
* The SiLU-gated producer silu(gate) * up -> q8_1 (gate page, ``main``: the MoE expert-ff
  site), in f64 with one rounding to f32, then the q8_1 step -- see ``oracle.c``.
* The KDA gated-norm producer the gate page names at the 64-head x 128 KDA width (``main``):
  per head, RMSNorm over the head's head_dim values times a shared gain, times the sigmoid
  output gate, in f64 with one rounding to f32, then the q8_1 step.  The page gives no
  formula; the reading is restated next to ``gated_rms_norm``.
* The load-time e4m3 -> Q8_0 requantisation the same page names as its ship path (QUESTION),
  in f32 with an fp16 block scale -- see ``oracle.c`` for the reading it takes.

Readings where the pages are silent are listed in the repository's design notes; the ones that
decide a value are restated next to the function that takes them.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
EPS = 1e-6


def build() -> None:
    """Compile ``oracle.c`` (plain C, IEEE, no contraction) into ``liboracle.so``."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                           "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_value.restype = ctypes.c_double
        lib.oracle_quantize_q8_1.argtypes = [vp, i32, i32, vp, vp]
        lib.oracle_quantize_q8_1.restype = i32
        lib.oracle_gemv_q8_0.argtypes = [vp, i64, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_gemv_q8_0.restype = i32
        lib.oracle_gemv_e4m3.argtypes = [vp, i64, f32, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_gemv_e4m3.restype = i32
        lib.oracle_gemv_e4m3_blk128.argtypes = [vp, i64, vp, i32, vp, vp, i32, i32, i32, i32,
                                                i32, vp, vp]
        lib.oracle_gemv_e4m3_blk128.restype = i32
        lib.oracle_silu_mul.argtypes = [vp, vp, i32, vp, vp]
        lib.oracle_silu_mul.restype = None
        lib.oracle_f32_to_fp16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_fp16.restype = ctypes.c_uint16
        lib.oracle_requant_q8_0.argtypes = [vp, i64, f32, vp, i32, vp, i64, i32, i32, i32, i32]
        lib.oracle_requant_q8_0.restype = i32
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------------- decoders

def e4m3_value(code: int) -> float:
    """OCP E4M3 value of one byte (NaN for 0x7F / 0xFF)."""
    return _load().oracle_e4m3_value(code)


def fp16_value(bits: int) -> float:
    """IEEE binary16 value of one bit pattern."""
    return _load().oracle_fp16_value(bits)


# ------------------------------------------------------------------------- producer

def silu_mul(gate: np.ndarray, up: np.ndarray):
    """h = silu(gate) * up: returns (h64, h32) with the shape of gate."""
    g = _c(gate, np.float32)
    u = _c(up, np.float32)
    assert g.shape == u.shape
    h64 = np.empty(g.shape, dtype=np.float64)
    h32 = np.empty(g.shape, dtype=np.float32)
    _load().oracle_silu_mul(g.ctypes.data, u.ctypes.data, g.size, h64.ctypes.data,
                            h32.ctypes.data)
    return h64, h32


def silu_mul_q8_1(gate: np.ndarray, up: np.ndarray):
    """The SiLU-gated chain: silu_mul then q8_1 of the f32 rows."""
    h64, h32 = silu_mul(gate, up)
    qs, d = quantize_q8_1(np.atleast_2d(h32))
    return {"h64": h64, "h32": h32, "qs": qs, "d": d}

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float = EPS):
    """RMSNorm of f32 rows x [nrows, ncols] with gain w [ncols].

    Returns (z64, z32, s64): the f64 result, its f32 rounding and the per-row f64 factor
    s = 1 / sqrt(mean(x^2) + eps).  eps is taken as an f32 constant (1e-6f), as the gate
    page passes it, then widened to f64.
    """
    x = np.atleast_2d(_c(x, np.float32))
    w = _c(w, np.float32)
    nrows, ncols = x.shape
    assert w.shape == (ncols,)
    eps64 = float(np.float32(eps))
    x64 = x.astype(np.float64)
    w64 = w.astype(np.float64)
    z64 = np.empty((nrows, ncols), dtype=np.float64)
    s64 = np.empty(nrows, dtype=np.float64)
    for r in range(nrows):
        ss = math.fsum(x64[r] * x64[r])
        s = 1.0 / math.sqrt(ss / ncols + eps64)
        s64[r] = s
        z64[r] = (x64[r] * w64) * s
    return z64, z64.astype(np.float32), s64


def _exp(t: float) -> float:
    """libm exp with IEEE overflow to +inf (Python's math.exp raises instead)."""
    try:
        return math.exp(t)
    except OverflowError:
        return math.inf


def gated_rms_norm(o: np.ndarray, g: np.ndarray, w: np.ndarray, head_dim: int,
                   eps: float = EPS):
    """KDA gated-norm of f32 rows o [nrows, ncols] with output gate g [nrows, ncols] and gain
    w [head_dim] (shared by all heads), ncols = heads * head_dim.

    The gate page (q8_fuse_gate.rs, module doc and ``main``) names the KDA gated-norm site at
    the KDA qkv width, 64 heads x 128 head_dim = 8192, as a producer site still on the unfused
    chain, but gives no formula.  Reading taken: the output stage of a KDA (Kimi delta
    attention) layer -- RMSNorm over each head's head_dim values (not over the whole row), the
    gain indexed by the position inside the head, then the sigmoid output gate applied after
    the norm, element by element.  eps is the f32 1e-6 the page passes to rms_norm, widened.
    For head h of row r, with j over that head's columns, all in f64:
      ss_h = sum_j o_j^2 (exactly rounded, math.fsum),  s_h = 1 / sqrt(ss_h / head_dim + eps)
      z64_j = ((o_j * w_{j mod head_dim}) * s_h) * (1 / (1 + exp(-g_j)))
    and the stored f32 is z32 = float32(z64).  Returns (z64, z32)."""
    o = np.atleast_2d(_c(o, np.float32))
    g = np.atleast_2d(_c(g, np.float32))
    w = _c(w, np.float32)
    nrows, ncols = o.shape
    assert g.shape == o.shape and w.shape == (head_dim,) and ncols % head_dim == 0
    eps64 = float(np.float32(eps))
    o64, g64, w64 = o.astype(np.float64), g.astype(np.float64), w.astype(np.float64)
    z64 = np.empty((nrows, ncols), dtype=np.float64)
    for r in range(nrows):
        for h in range(ncols // head_dim):
            sl = slice(h * head_dim, (h + 1) * head_dim)
            ss = math.fsum(o64[r, sl] * o64[r, sl])
            s = 1.0 / math.sqrt(ss / head_dim + eps64)
            gate = np.array([1.0 / (1.0 + _exp(-v)) for v in g64[r, sl]])
            z64[r, sl] = ((o64[r, sl] * w64) * s) * gate
    return z64, z64.astype(np.float32)


def gated_rmsnorm_q8_1(o: np.ndarray, g: np.ndarray, w: np.ndarray, head_dim: int,
                       eps: float = EPS):
    """The KDA gated-norm producer: gated_rms_norm then q8_1 of its f32 output."""
    z64, z32 = gated_rms_norm(o, g, w, head_dim, eps)
    qs, d = quantize_q8_1(z32)
    return {"z64": z64, "z32": z32, "qs": qs, "d": d}


def quantize_q8_1(z: np.ndarray):
    """q8_1 of f32 rows z [nrows, ncols]: (qs int8 [nrows, ncols], d f32 [nrows, ncols/32])."""
    z = np.atleast_2d(_c(z, np.float32))
    nrows, ncols = z.shape
    qs = np.empty((nrows, ncols), dtype=np.int8)
    d = np.empty((nrows, ncols // 32), dtype=np.float32)
    rc = _load().oracle_quantize_q8_1(z.ctypes.data, nrows, ncols, qs.ctypes.data, d.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_quantize_q8_1 refused its input ({rc}): "
                         + ("a block with no finite 1/d" if rc == -1 else "bad shape"))
    return qs, d


def rmsnorm_q8_1(x: np.ndarray, w: np.ndarray, eps: float = EPS):
    """The producer: RMSNorm then q8_1 of its f32 output.

    Returns dict with z64, z32, qs, d and d64 = max|z64| / 127 per block (for tolerances).
    """
    z64, z32, s64 = rms_norm(x, w, eps)
    qs, d = quantize_q8_1(z32)
    nrows, ncols = z64.shape
    d64 = np.abs(z64).reshape(nrows, ncols // 32, 32).max(axis=2) / 127.0
    return {"z64": z64, "z32": z32, "s64": s64, "qs": qs, "d": d, "d64": d64}


# --------------------------------------------------------------------------- GEMVs

def _gemv_out(m, out_f):
    y = np.full((m, out_f), np.nan, dtype=np.float64)
    A = np.full((m, out_f), np.nan, dtype=np.float64)
    return y, A


def _rows(rows, out_f):
    if rows is None:
        return 0, out_f
    r0, r1 = rows
    return int(r0), int(r1)


def _act(qs, d, in_f):
    qs = np.atleast_2d(_c(qs, np.int8))
    d = np.atleast_2d(_c(d, np.float32))
    m = qs.shape[0]
    assert qs.shape == (m, in_f) and d.shape == (m, in_f // 32)
    return qs, d, m


def gemv_q8_0(W, row_bytes, qs, d, in_f, out_f, rows=None):
    """Q8_0 GEMV. Returns (y, A), f64 [m, out_f]; rows outside ``rows`` are NaN."""
    W = _c(W, np.uint8)
    qs, d, m = _act(qs, d, in_f)
    assert W.size >= out_f * row_bytes
    y, A = _gemv_out(m, out_f)
    r0, r1 = _rows(rows, out_f)
    rc = _load().oracle_gemv_q8_0(W.ctypes.data, row_bytes, qs.ctypes.data, d.ctypes.data, m,
                                  in_f, out_f, r0, r1, y.ctypes.data, A.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemv_q8_0 refused its input ({rc})")
    return y, A


def gemv_e4m3(W, row_bytes, scale, qs, d, in_f, out_f, rows=None):
    """Per-tensor-scale e4m3 GEMV. Returns (y, A), f64 [m, out_f]."""
    W = _c(W, np.uint8)
    qs, d, m = _act(qs, d, in_f)
    assert W.size >= out_f * row_bytes
    y, A = _gemv_out(m, out_f)
    r0, r1 = _rows(rows, out_f)
    rc = _load().oracle_gemv_e4m3(W.ctypes.data, row_bytes, float(scale), qs.ctypes.data,
                                  d.ctypes.data, m, in_f, out_f, r0, r1, y.ctypes.data,
                                  A.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemv_e4m3 refused its input ({rc})")
    return y, A


def gemv_e4m3_blk128(W, row_bytes, grid, qs, d, in_f, out_f, rows=None):
    """Block-128-scaled e4m3 GEMV. Returns (y, A), f64 [m, out_f]."""
    W = _c(W, np.uint8)
    grid = _c(grid, np.float32)
    qs, d, m = _act(qs, d, in_f)
    grid_cols = (in_f + 127) // 128
    assert W.size >= out_f * row_bytes and grid.size == ((out_f + 127) // 128) * grid_cols
    y, A = _gemv_out(m, out_f)
    r0, r1 = _rows(rows, out_f)
    rc = _load().oracle_gemv_e4m3_blk128(W.ctypes.data, row_bytes, grid.ctypes.data, grid_cols,
                                         qs.ctypes.data, d.ctypes.data, m, in_f, out_f, r0, r1,
                                         y.ctypes.data, A.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemv_e4m3_blk128 refused its input ({rc})")
    return y, A


# ---------------------------------------------------------------------- requantiser

def f32_to_fp16(x: float) -> int:
    """binary16 bit pattern of an f32, round to nearest even."""
    return int(_load().oracle_f32_to_fp16(float(np.float32(x))))


def requant_q8_0(W, row_bytes, in_f, out_f, scale=None, grid=None, rows=None, q_row_bytes=None):
    """e4m3 rows -> ggml Q8_0 rows (per-tensor ``scale`` or block-128 ``grid``).

    Returns uint8 [out_f, q_row_bytes] (q_row_bytes defaults to in_f / 32 * 34); rows outside
    ``rows`` and bytes past each row's blocks are zero."""
    W = _c(W, np.uint8)
    assert (scale is None) != (grid is None)
    nb = in_f // 32
    qrb = nb * 34 if q_row_bytes is None else int(q_row_bytes)
    assert W.size >= out_f * row_bytes
    out = np.zeros((out_f, qrb), dtype=np.uint8)
    r0, r1 = _rows(rows, out_f)
    if grid is not None:
        grid = _c(grid, np.float32)
        grid_cols = (in_f + 127) // 128
        assert grid.size == ((out_f + 127) // 128) * grid_cols
        rc = _load().oracle_requant_q8_0(W.ctypes.data, row_bytes, 0.0, grid.ctypes.data,
                                         grid_cols, out.ctypes.data, qrb, in_f, out_f, r0, r1)
    else:
        rc = _load().oracle_requant_q8_0(W.ctypes.data, row_bytes, float(scale), None, 0,
                                         out.ctypes.data, qrb, in_f, out_f, r0, r1)
    if rc != 0:
        raise ValueError(f"oracle_requant_q8_0 refused its input ({rc})")
    return out
