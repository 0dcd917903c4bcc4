"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

Nothing here computes any step of the matvec path: the module only draws floats and bytes
from one xorshift64 stream per array (``synth.c`` documents the exact recipe).  The HIP
library and the CPU oracle both consume these arrays; neither is imported from here.

Seeds follow the fused-producer gate page (q8_fuse_gate.rs, ``run_shape``): x rows use
``0x9E3779B97F4A7C15 ^ ncols`` and the norm gain ``0xD1B54A32D192ED03 ^ ncols``; activation
row t of an m-row batch also xors ``t << 48`` so that row 0 is the m=1 input.  Weight planes
use the seeds of the GEMV bench page's synthesisers (gemv_e4m3_bench.rs, ``synth_e4m3``,
``synth_q8_0``, ``synth_blk_grid``) xor ``(out_f << 32) | in_f``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

SEED_X = 0x9E3779B97F4A7C15
SEED_W = 0xD1B54A32D192ED03
SEED_E4M3 = 0x12345678
SEED_Q8_0 = 0x9E3779B9
SEED_GRID = 0x5BF03635
_M64 = (1 << 64) - 1


def build() -> None:
    """Compile ``synth.c`` into ``libsynth.so`` next to this file."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        for name in ("synth_f32", "synth_e4m3", "synth_i8", "synth_grid", "synth_raw_u64"):
            getattr(lib, name).argtypes = [u64, vp, i64]
            getattr(lib, name).restype = None
        lib.synth_q8_0.argtypes = [u64, vp, i64, i64]
        lib.synth_q8_0.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def raw_u64(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_raw_u64(seed & _M64, _ptr(out), n)
    return out


def f32(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_f32(seed & _M64, _ptr(out), n)
    return out


def i8(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int8)
    _load().synth_i8(seed & _M64, _ptr(out), n)
    return out


def e4m3(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _load().synth_e4m3(seed & _M64, _ptr(out), n)
    return out


def x_rows(ncols: int, m: int = 1) -> np.ndarray:
    """Activation rows x[t, :] in [-4, 4), never 0; row 0 is the m=1 input."""
    out = np.empty((m, ncols), dtype=np.float32)
    for t in range(m):
        out[t] = f32(SEED_X ^ ncols ^ (t << 48), ncols)
    return out


def gain(ncols: int) -> np.ndarray:
    """RMSNorm gain vector w in [-4, 4), never 0."""
    return f32(SEED_W ^ ncols, ncols)


def _shape_seed(base: int, out_f: int, in_f: int) -> int:
    return (base ^ ((out_f << 32) | in_f)) & _M64


def e4m3_weights(out_f: int, in_f: int) -> np.ndarray:
    """Raw e4m3 plane [out_f, in_f], row stride in_f, no NaN codes."""
    out = np.empty((out_f, in_f), dtype=np.uint8)
    _load().synth_e4m3(_shape_seed(SEED_E4M3, out_f, in_f), _ptr(out), out.size)
    return out


def q8_0_weights(out_f: int, in_f: int) -> np.ndarray:
    """ggml Q8_0 rows [out_f, in_f/32*34]: int8 in [-127, 127], fp16 scales in [2^-8, 2^-4]."""
    assert in_f % 32 == 0
    out = np.empty((out_f, in_f // 32 * 34), dtype=np.uint8)
    _load().synth_q8_0(_shape_seed(SEED_Q8_0, out_f, in_f), _ptr(out), out_f, in_f)
    return out


def blk128_grid(out_f: int, in_f: int) -> np.ndarray:
    """f32 scale grid [ceil(out_f/128), ceil(in_f/128)], powers of two 2^-6 .. 2^-2."""
    g = np.empty(((out_f + 127) // 128, (in_f + 127) // 128), dtype=np.float32)
    _load().synth_grid(_shape_seed(SEED_GRID, out_f, in_f), _ptr(g), g.size)
    return g
