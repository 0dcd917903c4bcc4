"""Python binding of the gfx950 m=1 decode matvec library (``libfp8_gemv.so``).

Each function has the name and argument order of the C entry point in
``include/fp8_gemv.h``.  The binding only marshals arguments: it checks that every tensor
is a contiguous tensor of the right dtype on the current GPU and large enough for the sizes
passed (the C side cannot see buffer sizes), turns tensors into device pointers, takes the
current torch stream when none is given, and raises on a non-zero return code.  Every step of
the computation runs in the library's HIP kernels; there is no fallback of any kind, and
importing this package fails if the library has not been built.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the process's HIP runtime before the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8_gemv.so")

FP8GEMV_OK = 0
FP8GEMV_ERR_NULL = -1
FP8GEMV_ERR_SHAPE = -2
FP8GEMV_ERR_ROW_BYTES = -3
FP8GEMV_ERR_GRID = -4
FP8GEMV_ERR_ALIGN = -5
FP8GEMV_ERR_TOO_LARGE = -6
FP8GEMV_MAX_IN_F = 65536
FP8GEMV_MAX_M = 65535

EXPORTS = ("rms_norm_f32", "quantize_q8_1", "rmsnorm_q8_1", "silu_mul_f32", "silu_mul_q8_1",
           "gated_rms_norm_f32", "gated_rmsnorm_q8_1",
           "gemv_q8_0_q81", "gemv_e4m3_q81",
           "gemv_e4m3_blk128_q81", "gemv_q8_0_q81_mc", "gemv_e4m3_q81_mc",
           "gemv_e4m3_blk128_q81_mc", "requant_e4m3_q8_0", "requant_e4m3_blk128_q8_0",
           "fp8gemv_read_bytes", "fp8gemv_read_pattern", "fp8gemv_gemv_launch_info",
           "fp8gemv_strerror")


FP8GEMV_Q8_0 = 0
FP8GEMV_E4M3 = 1
FP8GEMV_E4M3_BLK128 = 2
FP8GEMV_Q8_0_MC = 3
FP8GEMV_E4M3_MC = 4
FP8GEMV_E4M3_BLK128_MC = 5
CONTAINERS = {"q8_0": FP8GEMV_Q8_0, "e4m3": FP8GEMV_E4M3, "blk128": FP8GEMV_E4M3_BLK128,
              "q8_0_mc": FP8GEMV_Q8_0_MC, "e4m3_mc": FP8GEMV_E4M3_MC,
              "blk128_mc": FP8GEMV_E4M3_BLK128_MC}


class LaunchInfo(ctypes.Structure):
    """fp8gemv_launch_info of the header."""
    _fields_ = [("grid_x", ctypes.c_uint32), ("grid_y", ctypes.c_uint32),
                ("workgroup_size", ctypes.c_uint32), ("lds_bytes", ctypes.c_uint32),
                ("kernel", ctypes.c_char_p), ("config", ctypes.c_char_p)]


class Fp8GemvError(RuntimeError):
    """A non-zero return code from the library."""

    def __init__(self, fn: str, rc: int, msg: str):
        super().__init__(f"{fn}: {msg} (rc={rc})")
        self.rc = rc


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()' or python fp8_gemv_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    sig = {
        "rms_norm_f32": [vp, vp, vp, i32, i32, f32, vp],
        "quantize_q8_1": [vp, vp, vp, i32, i32, vp],
        "rmsnorm_q8_1": [vp, vp, vp, vp, vp, i32, i32, f32, vp],
        "silu_mul_f32": [vp, vp, vp, i32, i32, vp],
        "silu_mul_q8_1": [vp, vp, vp, vp, vp, i32, i32, vp],
        "gated_rms_norm_f32": [vp, vp, vp, vp, i32, i32, i32, f32, vp],
        "gated_rmsnorm_q8_1": [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp],
        "gemv_q8_0_q81": [vp, i64, vp, vp, vp, i32, i32, i32, vp],
        "gemv_e4m3_q81": [vp, i64, f32, vp, vp, vp, i32, i32, i32, vp],
        "gemv_e4m3_blk128_q81": [vp, i64, vp, i32, vp, vp, vp, i32, i32, i32, vp],
        "gemv_q8_0_q81_mc": [vp, i64, vp, vp, vp, i32, i32, i32, vp],
        "gemv_e4m3_q81_mc": [vp, i64, f32, vp, vp, vp, i32, i32, i32, vp],
        "gemv_e4m3_blk128_q81_mc": [vp, i64, vp, i32, vp, vp, vp, i32, i32, i32, vp],
        "requant_e4m3_q8_0": [vp, i64, f32, vp, i64, i32, i32, vp],
        "requant_e4m3_blk128_q8_0": [vp, i64, vp, i32, vp, i64, i32, i32, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    lib.fp8gemv_read_bytes.argtypes = [vp, i64, vp, vp]
    lib.fp8gemv_read_bytes.restype = i32
    lib.fp8gemv_read_pattern.argtypes = [vp, i64, i32, i64, vp, vp]
    lib.fp8gemv_read_pattern.restype = i32
    lib.fp8gemv_gemv_launch_info.argtypes = [i32, vp, i64, i32, i32, i32,
                                             ctypes.POINTER(LaunchInfo)]
    lib.fp8gemv_gemv_launch_info.restype = i32
    lib.fp8gemv_strerror.argtypes = [i32]
    lib.fp8gemv_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    """The loaded C library (for callers that marshal pointers themselves)."""
    return _lib


def strerror(rc: int) -> str:
    return _lib.fp8gemv_strerror(int(rc)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise Fp8GemvError(fn, rc, strerror(rc))


def _stream(stream, dev=None) -> int:
    """The stream handle: the given one, else torch's current stream of the tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _run(name: str, dev, *args) -> None:
    """Call one entry point with the tensors' device current: the library launches on the
    current HIP device and raises per-device kernel attributes there."""
    fn = getattr(_lib, name)
    if dev is None:
        rc = fn(*args)
    else:
        with torch.cuda.device(dev):
            rc = fn(*args)
    _check(name, rc)


def _ptr(t, name: str, dtype, min_numel: int, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: has {t.numel()} elements, the sizes passed need {min_numel}")
    return t.data_ptr()


def _dev(t):
    return t.device if isinstance(t, torch.Tensor) else None


# ----------------------------------------------------------------------------- producer

def rms_norm_f32(x, w, z, ncols: int, nrows: int, eps: float = 1e-6, stream=None) -> None:
    """z[r, :] = x[r, :] * w / sqrt(mean(x[r, :]^2) + eps)  (first half of the chain)."""
    dev = _dev(x)
    _run("rms_norm_f32", dev,
         _ptr(x, "x", torch.float32, ncols * nrows, dev),
         _ptr(w, "w", torch.float32, ncols, dev),
         _ptr(z, "z", torch.float32, ncols * nrows, dev),
         ncols, nrows, eps, _stream(stream, dev))


def quantize_q8_1(z, qs, d, nrows: int, ncols: int, stream=None) -> None:
    """q8_1 of f32 rows: qs int8 [nrows, ncols], d f32 [nrows, ncols/32]."""
    dev = _dev(z)
    _run("quantize_q8_1", dev,
         _ptr(z, "z", torch.float32, ncols * nrows, dev),
         _ptr(qs, "qs", torch.int8, ncols * nrows, dev),
         _ptr(d, "d", torch.float32, (ncols // 32) * nrows, dev),
         nrows, ncols, _stream(stream, dev))


def rmsnorm_q8_1(x, w, z, qs, d, ncols: int, nrows: int, eps: float = 1e-6,
                 stream=None) -> None:
    """Fused producer: RMSNorm then q8_1 in one launch (z may be None)."""
    dev = _dev(x)
    _run("rmsnorm_q8_1", dev,
         _ptr(x, "x", torch.float32, ncols * nrows, dev),
         _ptr(w, "w", torch.float32, ncols, dev),
         _ptr(z, "z", torch.float32, ncols * nrows, dev),
         _ptr(qs, "qs", torch.int8, ncols * nrows, dev),
         _ptr(d, "d", torch.float32, (ncols // 32) * nrows, dev),
         ncols, nrows, eps, _stream(stream, dev))


def silu_mul_f32(gate, up, h, ncols: int, nrows: int, stream=None) -> None:
    """h = silu(gate) * up (first half of the SiLU-gated chain)."""
    dev = _dev(gate)
    n = ncols * nrows
    _run("silu_mul_f32", dev,
         _ptr(gate, "gate", torch.float32, n, dev),
         _ptr(up, "up", torch.float32, n, dev),
         _ptr(h, "h", torch.float32, n, dev),
         ncols, nrows, _stream(stream, dev))


def silu_mul_q8_1(gate, up, h, qs, d, ncols: int, nrows: int, stream=None) -> None:
    """Fused SiLU-gated producer: silu(gate) * up then q8_1 in one launch (h may be None)."""
    dev = _dev(gate)
    n = ncols * nrows
    _run("silu_mul_q8_1", dev,
         _ptr(gate, "gate", torch.float32, n, dev),
         _ptr(up, "up", torch.float32, n, dev),
         _ptr(h, "h", torch.float32, n, dev),
         _ptr(qs, "qs", torch.int8, n, dev),
         _ptr(d, "d", torch.float32, (ncols // 32) * nrows, dev),
         ncols, nrows, _stream(stream, dev))


def gated_rms_norm_f32(o, g, w, z, ncols: int, head_dim: int, nrows: int, eps: float = 1e-6,
                       stream=None) -> None:
    """KDA gated norm z = RMSNorm per head(o) * w * sigmoid(g) (first half of its chain)."""
    dev = _dev(o)
    n = ncols * nrows
    _run("gated_rms_norm_f32", dev,
         _ptr(o, "o", torch.float32, n, dev),
         _ptr(g, "g", torch.float32, n, dev),
         _ptr(w, "w", torch.float32, head_dim, dev),
         _ptr(z, "z", torch.float32, n, dev),
         ncols, head_dim, nrows, eps, _stream(stream, dev))


def gated_rmsnorm_q8_1(o, g, w, z, qs, d, ncols: int, head_dim: int, nrows: int,
                       eps: float = 1e-6, stream=None) -> None:
    """Fused KDA gated-norm producer: the gated norm then q8_1 in one launch (z may be None)."""
    dev = _dev(o)
    n = ncols * nrows
    _run("gated_rmsnorm_q8_1", dev,
         _ptr(o, "o", torch.float32, n, dev),
         _ptr(g, "g", torch.float32, n, dev),
         _ptr(w, "w", torch.float32, head_dim, dev),
         _ptr(z, "z", torch.float32, n, dev),
         _ptr(qs, "qs", torch.int8, n, dev),
         _ptr(d, "d", torch.float32, (ncols // 32) * nrows, dev),
         ncols, head_dim, nrows, eps, _stream(stream, dev))


# -------------------------------------------------------------------------------- GEMVs

def _w_numel(row_bytes: int, out_f: int, container_row: int) -> int:
    # the last row only needs its used bytes
    return (out_f - 1) * row_bytes + container_row if out_f >= 1 else 0


def gemv_q8_0_q81(W, row_bytes: int, qs, d, y, m: int, in_f: int, out_f: int,
                  stream=None, _entry="gemv_q8_0_q81") -> None:
    """y[m, out_f] = Q8_0 weight rows W times the q8_1 activation (qs, d)."""
    dev = _dev(W)
    _run(_entry, dev,
         _ptr(W, "W", torch.uint8, _w_numel(row_bytes, out_f, in_f // 32 * 34), dev), row_bytes,
         _ptr(qs, "qs", torch.int8, m * in_f, dev),
         _ptr(d, "d", torch.float32, m * (in_f // 32), dev),
         _ptr(y, "y", torch.float32, m * out_f, dev),
         m, in_f, out_f, _stream(stream, dev))


def gemv_e4m3_q81(W, row_bytes: int, scale: float, qs, d, y, m: int, in_f: int, out_f: int,
                  stream=None, _entry="gemv_e4m3_q81") -> None:
    """y[m, out_f] = scale * e4m3 weights W times the q8_1 activation (qs, d)."""
    dev = _dev(W)
    _run(_entry, dev,
         _ptr(W, "W", torch.uint8, _w_numel(row_bytes, out_f, in_f), dev), row_bytes, scale,
         _ptr(qs, "qs", torch.int8, m * in_f, dev),
         _ptr(d, "d", torch.float32, m * (in_f // 32), dev),
         _ptr(y, "y", torch.float32, m * out_f, dev),
         m, in_f, out_f, _stream(stream, dev))


def gemv_e4m3_blk128_q81(W, row_bytes: int, grid, grid_cols: int, qs, d, y, m: int, in_f: int,
                         out_f: int, stream=None, _entry="gemv_e4m3_blk128_q81") -> None:
    """y[m, out_f] = block-128-scaled e4m3 weights W times the q8_1 activation (qs, d)."""
    dev = _dev(W)
    _run(_entry, dev,
         _ptr(W, "W", torch.uint8, _w_numel(row_bytes, out_f, in_f), dev), row_bytes,
         _ptr(grid, "grid", torch.float32, ((out_f + 127) // 128) * grid_cols, dev), grid_cols,
         _ptr(qs, "qs", torch.int8, m * in_f, dev),
         _ptr(d, "d", torch.float32, m * (in_f // 32), dev),
         _ptr(y, "y", torch.float32, m * out_f, dev),
         m, in_f, out_f, _stream(stream, dev))


def gemv_q8_0_q81_mc(W, row_bytes: int, qs, d, y, m: int, in_f: int, out_f: int,
                     stream=None) -> None:
    """gemv_q8_0_q81 on the matrix cores (rows agree with it to rounding, not bit for bit)."""
    gemv_q8_0_q81(W, row_bytes, qs, d, y, m, in_f, out_f, stream, _entry="gemv_q8_0_q81_mc")


def gemv_e4m3_q81_mc(W, row_bytes: int, scale: float, qs, d, y, m: int, in_f: int, out_f: int,
                     stream=None) -> None:
    """gemv_e4m3_q81 on the matrix cores (rows agree with it to rounding, not bit for bit)."""
    gemv_e4m3_q81(W, row_bytes, scale, qs, d, y, m, in_f, out_f, stream,
                  _entry="gemv_e4m3_q81_mc")


def gemv_e4m3_blk128_q81_mc(W, row_bytes: int, grid, grid_cols: int, qs, d, y, m: int,
                            in_f: int, out_f: int, stream=None) -> None:
    """gemv_e4m3_blk128_q81 on the matrix cores (rows agree with it to rounding, not bit for
    bit)."""
    gemv_e4m3_blk128_q81(W, row_bytes, grid, grid_cols, qs, d, y, m, in_f, out_f, stream,
                         _entry="gemv_e4m3_blk128_q81_mc")


# --------------------------------------------------------------------------- requantiser

def _q_numel(q_row_bytes: int, out_f: int, in_f: int) -> int:
    return (out_f - 1) * q_row_bytes + in_f // 32 * 34 if out_f >= 1 else 0


def requant_e4m3_q8_0(W, row_bytes: int, scale: float, Wq, q_row_bytes: int, in_f: int,
                      out_f: int, stream=None) -> None:
    """Load-time e4m3 (per-tensor scale) -> Q8_0 rows in Wq (uint8)."""
    dev = _dev(W)
    _run("requant_e4m3_q8_0", dev,
         _ptr(W, "W", torch.uint8, _w_numel(row_bytes, out_f, in_f), dev), row_bytes, scale,
         _ptr(Wq, "Wq", torch.uint8, _q_numel(q_row_bytes, out_f, in_f), dev), q_row_bytes,
         in_f, out_f, _stream(stream, dev))


def requant_e4m3_blk128_q8_0(W, row_bytes: int, grid, grid_cols: int, Wq, q_row_bytes: int,
                             in_f: int, out_f: int, stream=None) -> None:
    """Load-time block-128 e4m3 -> Q8_0 rows in Wq (uint8)."""
    dev = _dev(W)
    _run("requant_e4m3_blk128_q8_0", dev,
         _ptr(W, "W", torch.uint8, _w_numel(row_bytes, out_f, in_f), dev), row_bytes,
         _ptr(grid, "grid", torch.float32, ((out_f + 127) // 128) * grid_cols, dev), grid_cols,
         _ptr(Wq, "Wq", torch.uint8, _q_numel(q_row_bytes, out_f, in_f), dev), q_row_bytes,
         in_f, out_f, _stream(stream, dev))


def fp8gemv_read_bytes(buf, nbytes: int, sink, stream=None) -> None:
    """Measurement aid: stream nbytes of buf with the GEMVs' load pattern (no result)."""
    dev = _dev(buf)
    _run("fp8gemv_read_bytes", dev,
         _ptr(buf, "buf", torch.uint8, nbytes, dev), nbytes,
         _ptr(sink, "sink", torch.int32, 1, dev), _stream(stream, dev))


# Load patterns of fp8gemv_read_pattern (the FP8GEMV_READ_* constants of the header).
FP8GEMV_READ_CHUNK8K = 0
FP8GEMV_READ_CHUNK16K = 1
FP8GEMV_READ_WG8 = 2
FP8GEMV_READ_WG16 = 3
FP8GEMV_READ_PERSISTENT = 4
FP8GEMV_READ_CACHED = 5
FP8GEMV_READ_ROWS_1K = 6
FP8GEMV_READ_ROWS_816 = 7
FP8GEMV_READ_EMPTY = 8
FP8GEMV_READ_ONE_WAVE = 9
FP8GEMV_READ_ROWS_ALIGNED = 10
FP8GEMV_READ_LINE_WINDOWS = 11
FP8GEMV_READ_NUM_PATTERNS = 12
READ_PATTERNS = {"chunk8k": FP8GEMV_READ_CHUNK8K, "chunk16k": FP8GEMV_READ_CHUNK16K,
                 "wg8": FP8GEMV_READ_WG8, "wg16": FP8GEMV_READ_WG16,
                 "persistent": FP8GEMV_READ_PERSISTENT, "cached": FP8GEMV_READ_CACHED,
                 "rows_1k": FP8GEMV_READ_ROWS_1K, "rows_816": FP8GEMV_READ_ROWS_816,
                 "empty": FP8GEMV_READ_EMPTY, "one_wave": FP8GEMV_READ_ONE_WAVE,
                 "rows_aligned": FP8GEMV_READ_ROWS_ALIGNED,
                 "line_windows": FP8GEMV_READ_LINE_WINDOWS}


def fp8gemv_read_pattern(buf, nbytes: int, pattern: str, sink, row_bytes: int = 0,
                         stream=None) -> None:
    """Measurement aid: stream nbytes of buf in one of READ_PATTERNS (no result)."""
    dev = _dev(buf)
    _run("fp8gemv_read_pattern", dev,
         _ptr(buf, "buf", torch.uint8, nbytes, dev), nbytes, READ_PATTERNS[pattern], row_bytes,
         _ptr(sink, "sink", torch.int32, 1, dev), _stream(stream, dev))


def gemv_launch_info(container: str, row_bytes: int, m: int, in_f: int, out_f: int,
                     w_align: int = 256) -> dict:
    """What the GEMV of `container` launches for these arguments (no device work): grid in
    workgroups, threads per workgroup, dynamic LDS bytes, kernel family and configuration.
    `w_align` is the weight pointer's alignment (it decides the Q8_0 fast path)."""
    info = LaunchInfo()
    rc = _lib.fp8gemv_gemv_launch_info(CONTAINERS[container], w_align, row_bytes, m, in_f, out_f,
                                       ctypes.byref(info))
    if rc != 0:
        raise Fp8GemvError("fp8gemv_gemv_launch_info", rc, strerror(rc))
    return {"grid_x": info.grid_x, "grid_y": info.grid_y, "workgroup_size": info.workgroup_size,
            "lds_bytes": info.lds_bytes, "kernel": info.kernel.decode(),
            "config": info.config.decode()}


# ------------------------------------------------------------------------- byte counts

def e4m3_weight_bytes(out_f: int, in_f: int) -> int:
    """Weight-plane bytes of a raw e4m3 matrix: one byte per weight."""
    return out_f * in_f


def q8_0_weight_bytes(out_f: int, in_f: int) -> int:
    """Weight-plane bytes of a Q8_0 matrix: 34 bytes per 32 weights."""
    return out_f * (in_f // 32) * 34


def blk128_grid_bytes(out_f: int, in_f: int) -> int:
    """Bytes of the f32 [ceil(out_f/128), ceil(in_f/128)] scale grid."""
    return 4 * ((out_f + 127) // 128) * ((in_f + 127) // 128)
