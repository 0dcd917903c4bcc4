"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each test ties one oracle function to something independent of it: values the pages print
(golden fixtures, each with its citation), a library routine that implements the same
definition (torch's float8_e4m3fn cast, numpy's float16, torch's rms_norm, numpy matmul),
exact rational brute force on tiny inputs, closed forms and invariants.  The cases are
chosen so that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, the wrong rounding rule) fails at least one of them.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import read_blocks, read_points


# ----------------------------------------------------------------------------- decoders

def _same(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e4m3_golden_points():
    pts = read_points("e4m3_points.txt")
    assert len(pts) >= 10
    for code, want in pts:
        assert _same(oracle.e4m3_value(code), want), hex(code)


def test_e4m3_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e4m3_value(c), float(lib[c])), hex(c)


def test_fp16_golden_points():
    pts = read_points("fp16_points.txt")
    for bits, want in pts:
        assert _same(oracle.fp16_value(bits), want), hex(bits)


def test_fp16_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    lib = bits.view(np.float16).astype(np.float64)
    for b in range(65536):
        assert _same(oracle.fp16_value(b), float(lib[b])), hex(b)


# ---------------------------------------------------------------------------- quantiser

def test_q8_1_golden_blocks():
    blocks = read_blocks("q8_1_blocks.txt")
    assert {"unit_scale_ties", "pow2_scaled", "all_zero", "constant", "negative_max",
            "reciprocal_not_division"} <= set(blocks)
    for name, blk in blocks.items():
        z = np.array(blk["z"], dtype=np.float32)
        assert z.shape == (32,) and np.all(z.astype(np.float64) == np.array(blk["z"])), name
        qs, d = oracle.quantize_q8_1(z[None, :])
        assert qs[0].tolist() == blk["q"], name
        if "d" in blk:
            assert float(d[0, 0]) == blk["d"], name


def _blocks(seed, nblocks):
    return synth.f32(seed, nblocks * 32).reshape(nblocks, 32)


def test_q8_1_scale_is_correctly_rounded_amax_over_127():
    z = _blocks(11, 2000)
    qs, d = oracle.quantize_q8_1(z.reshape(1, -1))
    d = d.reshape(-1)
    amax = np.abs(z).max(axis=1)
    for i in range(0, 2000, 7):
        exact = Fraction(float(amax[i])) / 127
        got = Fraction(float(d[i]))
        for nb in (np.nextafter(d[i], np.float32(np.inf)), np.nextafter(d[i], np.float32(0))):
            assert abs(got - exact) <= abs(Fraction(float(nb)) - exact)


def test_q8_1_invariants():
    z = _blocks(12, 4000)
    # make some blocks small, some spread over binades, one negative-dominant
    z[::3] *= np.float32(2.0 ** -12)
    z[1::5, 7] = np.float32(-9.5)
    qs, d = oracle.quantize_q8_1(z.reshape(1, -1))
    qs = qs.reshape(-1, 32).astype(np.int64)
    d = d.reshape(-1).astype(np.float64)
    z64 = z.astype(np.float64)
    assert np.all(np.abs(qs) <= 127)
    arg = np.abs(z).argmax(axis=1)
    rows = np.arange(len(z))
    assert np.all(qs[rows, arg] == np.sign(z64[rows, arg]) * 127)
    # q is z/d to the nearest integer (the f32 product z * (1/d) is within a few ulps of z/d)
    err = np.abs(z64 / d[:, None] - qs)
    assert err.max() <= 0.5 + 1e-4
    # a sign is never flipped
    assert np.all(qs * np.sign(z64) >= 0)
    # rows of a 2-D call are independent
    z2 = z[:64].reshape(2, 1024)
    q2, d2 = oracle.quantize_q8_1(z2)
    for r in range(2):
        qr, dr = oracle.quantize_q8_1(z2[r:r + 1])
        assert np.array_equal(q2[r], qr[0]) and np.array_equal(d2[r], dr[0])


@pytest.mark.parametrize("k", [-20, -7, -1, 1, 5, 30])
def test_q8_1_power_of_two_scaling(k):
    z = _blocks(13, 500)
    q0, d0 = oracle.quantize_q8_1(z.reshape(1, -1))
    zs = (z.astype(np.float64) * 2.0 ** k).astype(np.float32)
    q1, d1 = oracle.quantize_q8_1(zs.reshape(1, -1))
    assert np.array_equal(q0, q1)
    assert np.array_equal(d1.astype(np.float64), d0.astype(np.float64) * 2.0 ** k)


# ------------------------------------------------------------------------------ RMSNorm

EPS32 = float(np.float32(1e-6))


@pytest.mark.parametrize("ncols", [32, 1536, 4096, 8192])
def test_rms_norm_against_torch_f64(ncols):
    x = synth.x_rows(ncols, 3)
    w = synth.gain(ncols)
    z64, z32, s64 = oracle.rms_norm(x, w)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (ncols,),
                                       weight=torch.from_numpy(w).double(), eps=EPS32).numpy()
    assert np.all(np.abs(z64 - ref) <= 1e-14 * np.abs(ref) + 1e-300)
    assert np.array_equal(z32, z64.astype(np.float32))


@pytest.mark.parametrize("c", [2.0 ** -10, 0.75, -3.5])
def test_rms_norm_constant_row_closed_form(c):
    # x = c everywhere, w = 1: mean(x^2) = c^2 and z = c / sqrt(c^2 + eps).  The 2^-10 case
    # makes eps (1e-6f) comparable to c^2 = 9.5e-7, so where eps enters is visible.
    n = 256
    x = np.full((1, n), c, dtype=np.float32)
    w = np.ones(n, dtype=np.float32)
    z64, _, _ = oracle.rms_norm(x, w)
    getcontext().prec = 50
    dc = Decimal(c)
    want = float(dc / (dc * dc + Decimal(EPS32)).sqrt())
    assert np.all(np.abs(z64 - want) <= 4e-16 * abs(want))


def test_rms_norm_invariants():
    n = 4096
    x = synth.x_rows(n, 2)
    w = synth.gain(n)
    z64, _, s64 = oracle.rms_norm(x, w)
    # column permutation commutes (the exactly rounded sum does not depend on order)
    perm = np.random.default_rng(5).permutation(n)
    zp, _, sp = oracle.rms_norm(x[:, perm], w[perm])
    assert np.array_equal(zp, z64[:, perm]) and np.array_equal(sp, s64)
    # the gain enters linearly
    z2, _, _ = oracle.rms_norm(x, (w.astype(np.float64) * 2).astype(np.float32))
    assert np.array_equal(z2, 2 * z64)
    # mean((z / w)^2) = ms / (ms + eps), ms = mean(x^2)
    for r in range(2):
        ms = math.fsum(x[r].astype(np.float64) ** 2) / n
        got = np.mean((z64[r] / w.astype(np.float64)) ** 2)
        assert abs(got - ms / (ms + EPS32)) <= 1e-12
    # rows are independent
    z1, _, _ = oracle.rms_norm(x[1:2], w)
    assert np.array_equal(z1[0], z64[1])


# -------------------------------------------------------------------------------- GEMVs

def _e4m3_lib(W):
    return torch.from_numpy(np.ascontiguousarray(W)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _q8_0_lib(Wq, in_f):
    out_f = Wq.shape[0]
    nb = in_f // 32
    blk = Wq[:, :nb * 34].reshape(out_f, nb, 34)
    scale = blk[:, :, 0:2].copy().view(np.float16).astype(np.float64).reshape(out_f, nb)
    q = blk[:, :, 2:].view(np.int8).astype(np.float64)
    return (q * scale[:, :, None]).reshape(out_f, in_f)


def _act(in_f, m, seed):
    x = np.stack([synth.f32(seed + t, in_f) for t in range(m)])
    return oracle.quantize_q8_1(x)


def _dequant(kind, in_f, out_f, seed):
    """Weights of one container and their values via library decoders (f64 [out_f, in_f])."""
    if kind == "q8_0":
        Wq = synth.q8_0_weights(out_f, in_f)
        return Wq, _q8_0_lib(Wq, in_f), None
    W = synth.e4m3(seed, out_f * in_f).reshape(out_f, in_f)
    vals = _e4m3_lib(W)
    if kind == "e4m3":
        return W, vals * 2.0 ** -4, None
    g = synth.blk128_grid(out_f, in_f)
    gexp = np.repeat(np.repeat(g.astype(np.float64), 128, 0), 128, 1)[:out_f, :in_f]
    return W, vals * gexp, g


def _run(kind, W, grid, qs, d, in_f, out_f, rows=None):
    if kind == "q8_0":
        return oracle.gemv_q8_0(W, W.shape[1], qs, d, in_f, out_f, rows)
    if kind == "e4m3":
        return oracle.gemv_e4m3(W, in_f, 2.0 ** -4, qs, d, in_f, out_f, rows)
    return oracle.gemv_e4m3_blk128(W, in_f, grid, qs, d, in_f, out_f, rows)


KINDS = ["q8_0", "e4m3", "blk128"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("out_f,in_f,m", [(1, 32, 1), (3, 96, 2), (130, 160, 1), (131, 288, 2)])
def test_gemv_exact_rational_bruteforce(kind, out_f, in_f, m):
    W, w_hat, grid = _dequant(kind, in_f, out_f, seed=100 + in_f)
    qs, d = _act(in_f, m, seed=200 + out_f)
    y, A = _run(kind, W, grid, qs, d, in_f, out_f)
    a_hat = [[Fraction(float(d[t, k // 32])) * int(qs[t, k]) for k in range(in_f)]
             for t in range(m)]
    rows = range(out_f) if out_f <= 3 else [0, 1, 63, 127, 128, 129, out_f - 1]
    for t in range(m):
        for r in rows:
            terms = [Fraction(float(w_hat[r, k])) * a_hat[t][k] for k in range(in_f)]
            exact = sum(terms)
            aabs = sum(abs(v) for v in terms)
            tol = Fraction(in_f) * Fraction(1, 2 ** 52) * aabs
            assert abs(Fraction(float(y[t, r])) - exact) <= tol, (kind, t, r)
            assert abs(Fraction(float(A[t, r])) - aabs) <= tol, (kind, t, r)


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_against_numpy_matmul(kind):
    out_f, in_f, m = 257, 640, 2
    W, w_hat, grid = _dequant(kind, in_f, out_f, seed=7)
    qs, d = _act(in_f, m, seed=8)
    a_hat = qs.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    ref = a_hat @ w_hat.T
    y, A = _run(kind, W, grid, qs, d, in_f, out_f)
    assert np.all(np.abs(y - ref) <= 1e-12 * A)
    assert np.all(A >= np.abs(y))


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_one_hot_activation_reads_one_column(kind):
    out_f, in_f = 300, 384
    W, w_hat, grid = _dequant(kind, in_f, out_f, seed=9)
    for k0 in (0, 31, 32, 127, 128, 200, in_f - 1):
        qs = np.zeros((1, in_f), dtype=np.int8)
        qs[0, k0] = 1
        d = np.ones((1, in_f // 32), dtype=np.float32)
        y, A = _run(kind, W, grid, qs, d, in_f, out_f)
        assert np.array_equal(y[0], w_hat[:, k0]), (kind, k0)
        assert np.array_equal(A[0], np.abs(w_hat[:, k0]))


def test_gemv_q8_0_page_scale_bytes():
    # gemv_e4m3_bench.rs, synth_q8_0: bytes 0x00, 0x14 at the block head are f16 2^-10.
    in_f = 64
    W = np.zeros((1, 68), dtype=np.uint8)
    for b in range(2):
        W[0, 34 * b] = 0x00
        W[0, 34 * b + 1] = 0x14
        W[0, 34 * b + 2: 34 * b + 34] = np.arange(1, 33, dtype=np.uint8) * (1 + b)
    qs = np.ones((1, in_f), dtype=np.int8)
    d = np.ones((1, 2), dtype=np.float32)
    y, _ = oracle.gemv_q8_0(W, 68, qs, d, in_f, 1)
    assert y[0, 0] == 2.0 ** -10 * (528 + 2 * 528)


def test_gemv_constant_grid_equals_per_tensor():
    out_f, in_f = 300, 640
    W = synth.e4m3(21, out_f * in_f).reshape(out_f, in_f)
    qs, d = _act(in_f, 2, seed=22)
    grid = np.full(((out_f + 127) // 128, (in_f + 127) // 128), 2.0 ** -3, dtype=np.float32)
    yb, Ab = oracle.gemv_e4m3_blk128(W, in_f, grid, qs, d, in_f, out_f)
    ye, Ae = oracle.gemv_e4m3(W, in_f, 2.0 ** -3, qs, d, in_f, out_f)
    assert np.array_equal(yb, ye) and np.array_equal(Ab, Ae)


def test_gemv_all_ones_weights_sum_the_activation():
    out_f, in_f = 5, 512
    W = np.full((out_f, in_f), 0x38, dtype=np.uint8)  # e4m3 1.0
    qs, d = _act(in_f, 1, seed=23)
    y, _ = oracle.gemv_e4m3(W, in_f, 1.0, qs, d, in_f, out_f)
    want = math.fsum(float(d[0, k // 32]) * int(qs[0, k]) for k in range(in_f))
    assert np.all(np.abs(y[0] - want) <= 1e-13 * abs(want))


def test_gemv_row_stride_and_row_range():
    out_f, in_f, pad = 40, 256, 48
    W = synth.e4m3(31, out_f * in_f).reshape(out_f, in_f)
    Wp = np.zeros((out_f, in_f + pad), dtype=np.uint8)
    Wp[:, :in_f] = W
    Wp[:, in_f:] = 0x7F  # padding is never read (it would be refused as NaN)
    qs, d = _act(in_f, 1, seed=32)
    y, A = oracle.gemv_e4m3(W, in_f, 0.5, qs, d, in_f, out_f)
    yp, Ap = oracle.gemv_e4m3(Wp, in_f + pad, 0.5, qs, d, in_f, out_f)
    assert np.array_equal(y, yp)
    ys, _ = oracle.gemv_e4m3(W, in_f, 0.5, qs, d, in_f, out_f, rows=(10, 17))
    assert np.array_equal(ys[0, 10:17], y[0, 10:17]) and np.all(np.isnan(ys[0, :10]))


def test_gemv_refuses_nan_codes():
    out_f, in_f = 2, 64
    W = np.full((out_f, in_f), 0x38, dtype=np.uint8)
    W[1, 5] = 0xFF
    qs, d = _act(in_f, 1, seed=1)
    with pytest.raises(ValueError):
        oracle.gemv_e4m3(W, in_f, 1.0, qs, d, in_f, out_f)
    Wq = np.zeros((1, 34), dtype=np.uint8)
    Wq[0, 1] = 0x7C  # f16 +inf
    with pytest.raises(ValueError):
        oracle.gemv_q8_0(Wq, 34, qs[:, :32], d[:, :1], 32, 1)


# --------------------------------------------------------------------- requantiser
# e4m3 -> Q8_0 at load (gemv_e4m3_bench.rs, QUESTION: the ship path dequantises FP8 checkpoints
# to a Q8_0 slab).  The page gives no formula; the oracle takes the q8_1 block rule (id = 1/d,
# q = round(v * id)) with an fp16 scale.  Pinned by hand-worked blocks (three of them hold an
# element at half the block maximum, where the reciprocal and a plain division round apart),
# numpy's binary16 rounding, exact rationals and bounds.

def _read_requant_blocks():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "q8_0_requant_blocks.txt")
    blocks, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "block":
            cur = {"name": rest[0], "S": float.fromhex(rest[1]) if "0x" in rest[1] else float(rest[1])}
            blocks.append(cur)
        elif key == "codes":
            cur["codes"] = [int(t, 16) for t in rest]
        elif key == "scale":
            cur["scale"] = int(rest[0], 16)
        elif key == "q":
            cur["q"] = [int(t) for t in rest]
    return blocks


def test_requant_golden_blocks():
    blocks = _read_requant_blocks()
    assert len(blocks) >= 8
    for blk in blocks:
        W = np.array([blk["codes"]], dtype=np.uint8)
        out = oracle.requant_q8_0(W, 32, 32, 1, scale=blk["S"])[0]
        assert int(out[0]) | (int(out[1]) << 8) == blk["scale"], blk["name"]
        assert out[2:].view(np.int8).tolist() == blk["q"], blk["name"]


def test_f32_to_fp16_against_numpy():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    edge = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e9, 2.0 ** -14, 2.0 ** -24,
                     2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                     1.0 + 3 * 2.0 ** -11, 448 / 127, -3.25e-6], dtype=np.float32)
    for v in np.concatenate([vals[:20000], edge]):
        want = int(np.array([v], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f32_to_fp16(float(v)) == want, repr(v)


def _exact_block_checks(codes, S, out_block):
    """Stored scale = binary16 nearest the exact amax / 127 (up to f32 double rounding);
    q = rha(v * 127 / amax) unless that ratio sits within 2^-20 of a tie."""
    v = [Fraction(oracle.e4m3_value(c)) * Fraction(S) for c in codes]
    amax = max(abs(x) for x in v)
    h = int(out_block[0]) | (int(out_block[1]) << 8)
    q = out_block[2:].view(np.int8).tolist()
    if amax == 0:
        assert h == 0 and q == [0] * 32
        return
    d = amax / 127
    got = Fraction(oracle.fp16_value(h))
    e = math.floor(math.log2(d)) if d >= Fraction(1, 2 ** 14) else -14
    spacing = Fraction(2) ** (e - 10)
    assert abs(got - d) <= spacing / 2 * (1 + Fraction(1, 2 ** 12)), (h, float(d))
    for x, qi in zip(v, q):
        r = x / d
        a = abs(r)
        frac = a - math.floor(a)
        want = (math.floor(a) + (1 if frac >= Fraction(1, 2) else 0)) * (1 if r >= 0 else -1)
        if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20):
            assert abs(qi - want) <= 1
        else:
            assert qi == want, (float(r), qi)
    # the largest magnitude maps to +-127 with its sign
    i = max(range(32), key=lambda k: abs(v[k]))
    assert q[i] == (127 if v[i] > 0 else -127)


def test_requant_exact_rational_per_tensor():
    out_f, in_f = 6, 256
    W = synth.e4m3_weights(out_f, in_f)
    for S in (1.0, 2.0 ** -4, 0.3):
        Q = oracle.requant_q8_0(W, in_f, in_f, out_f, scale=S)
        for r in range(out_f):
            for b in range(in_f // 32):
                codes = W[r, 32 * b:32 * b + 32].tolist()
                Sf = float(np.float32(S))
                if S == 0.3:
                    # v = fl32(e4m3 * S) is not exact here; check against the rounded products
                    v32 = [float(np.float32(oracle.e4m3_value(c)) * np.float32(S)) for c in codes]
                    amax = max(abs(x) for x in v32)
                    h = int(Q[r, 34 * b]) | (int(Q[r, 34 * b + 1]) << 8)
                    assert abs(oracle.fp16_value(h) - amax / 127) <= amax / 127 * 2.0 ** -10
                    continue
                _exact_block_checks(codes, Sf, Q[r, 34 * b:34 * b + 34])


def test_requant_blk128_takes_the_tile_scale():
    out_f, in_f = 130, 384  # two row tiles, three column tiles
    W = synth.e4m3_weights(out_f, in_f)
    grid = synth.blk128_grid(out_f, in_f)
    Q = oracle.requant_q8_0(W, in_f, in_f, out_f, grid=grid)
    for r in (0, 77, 127, 128, 129):
        for b in range(in_f // 32):
            S = float(grid[r // 128, (32 * b) // 128])
            _exact_block_checks(W[r, 32 * b:32 * b + 32].tolist(), S, Q[r, 34 * b:34 * b + 34])
    # the same bytes under a per-tensor scale equal to one tile's value give that tile's blocks
    assert grid[0, 1] != grid[0, 0]
    Q1 = oracle.requant_q8_0(W, in_f, in_f, out_f, scale=float(grid[0, 1]))
    assert np.array_equal(Q1[:128, 34 * 4:34 * 8], Q[:128, 34 * 4:34 * 8])
    assert not np.array_equal(Q1[:128, :34 * 4], Q[:128, :34 * 4])


def test_requant_dequant_error_and_gemv_consistency():
    out_f, in_f = 40, 512
    W = synth.e4m3_weights(out_f, in_f)
    S = 2.0 ** -4
    Q = oracle.requant_q8_0(W, in_f, in_f, out_f, scale=S)
    nb = in_f // 32
    what = np.zeros((out_f, in_f))
    wq = np.zeros((out_f, in_f))
    err_bound = np.zeros((out_f, in_f))
    for r in range(out_f):
        for b in range(nb):
            blk = Q[r, 34 * b:34 * b + 34]
            d16 = oracle.fp16_value(int(blk[0]) | (int(blk[1]) << 8))
            q = blk[2:].view(np.int8).astype(np.float64)
            v = np.array([oracle.e4m3_value(c) for c in W[r, 32 * b:32 * b + 32]]) * S
            d = np.abs(v).max() / 127
            what[r, 32 * b:32 * b + 32] = v
            wq[r, 32 * b:32 * b + 32] = d16 * q
            err_bound[r, 32 * b:32 * b + 32] = d / 2 * (1 + 1e-6) + 127 * abs(d16 - d)
    assert np.all(np.abs(wq - what) <= err_bound)
    # the Q8_0 GEMV over the requantised rows differs from the e4m3 GEMV by at most the
    # propagated dequantisation error
    x = synth.x_rows(in_f, 1)
    qs, dd = oracle.quantize_q8_1(x)
    y8, _ = oracle.gemv_q8_0(Q, nb * 34, qs, dd, in_f, out_f)
    ye, _ = oracle.gemv_e4m3(W, in_f, S, qs, dd, in_f, out_f)
    a_hat = (np.repeat(dd.astype(np.float64), 32, axis=1) * qs.astype(np.float64))[0]
    bound = (err_bound * np.abs(a_hat)).sum(axis=1)
    assert np.all(np.abs(y8[0] - ye[0]) <= bound * (1 + 1e-9) + 1e-12)


def test_requant_refuses_nan_and_bad_shapes():
    W = np.zeros((1, 64), dtype=np.uint8)
    W[0, 40] = 0x7F
    with pytest.raises(ValueError):
        oracle.requant_q8_0(W, 64, 64, 1, scale=1.0)
    with pytest.raises(ValueError):
        oracle.requant_q8_0(np.zeros((1, 64), np.uint8), 64, 64, 1, scale=float("inf"))


# --------------------------------------------------------------- SiLU-gated producer
# silu(gate) * up (q8_fuse_gate.rs `main`: the MoE expert-ff activation site).  Pinned by
# torch's silu, high-precision Decimal evaluation, the odd-part identity and exact scaling.

def test_silu_mul_against_torch_f64():
    g = synth.f32(11, 4096)
    u = synth.f32(12, 4096)
    h64, h32 = oracle.silu_mul(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))) *
           torch.from_numpy(u.astype(np.float64))).numpy()
    assert np.allclose(h64, ref, rtol=4e-16, atol=0)
    assert np.array_equal(h32, h64.astype(np.float32))


def test_silu_mul_closed_forms_decimal():
    getcontext().prec = 60
    gs = np.array([0.0, 1.0, -1.0, 0.5, -3.75, 3.9999998, -0.0009765625, 20.0, -20.0, 40.0],
                  dtype=np.float32)
    us = np.array([1.0, 2.0, -0.75, 3.0, 1.0, -4.0, 1.5, 1.0, 1.0, 0.25], dtype=np.float32)
    h64, _ = oracle.silu_mul(gs, us)
    for g, u, h in zip(gs.tolist(), us.tolist(), h64.tolist()):
        gd = Decimal(g)
        want = gd / (1 + (-gd).exp()) * Decimal(u)
        if want == 0:
            assert h == 0.0
        else:
            assert abs(Decimal(h) - want) <= abs(want) * Decimal(2) ** -50, (g, u, h, want)


def test_silu_odd_part_identity_and_scaling():
    g = synth.f32(13, 2048)
    one = np.ones_like(g)
    hp, _ = oracle.silu_mul(g, one)
    hn, _ = oracle.silu_mul(-g, one)
    # silu(g) - silu(-g) = g
    assert np.allclose(hp - hn, g.astype(np.float64), rtol=1e-14, atol=1e-15)
    u = synth.f32(14, 2048)
    h1, _ = oracle.silu_mul(g, u)
    h2, _ = oracle.silu_mul(g, 2 * u)  # doubling is exact in f32 and f64
    assert np.array_equal(h2, 2 * h1)


# ------------------------------------------------------------ KDA gated-norm producer
# The gate page names the KDA gated-norm site (64 heads x 128 head_dim = 8192) without a
# formula; the oracle reads it as per-head RMSNorm x gain x sigmoid(gate), in f64.  Pinned by
# torch (rms_norm over each head reshaped as its own row, times torch.sigmoid), a 50-digit
# Decimal evaluation, the saturated and zero gates (exact reductions to the plain per-head
# RMSNorm and its half), head independence and the sigmoid's symmetry.

def _gated_inputs(ncols, head_dim, nrows=2, seed=21):
    o = np.stack([synth.f32(seed + r, ncols) for r in range(nrows)])
    g = np.stack([synth.f32(seed + 100 + r, ncols) for r in range(nrows)])
    return o, g, synth.gain(head_dim)


@pytest.mark.parametrize("head_dim", [32, 64, 128, 256])
def test_gated_norm_against_torch_f64(head_dim):
    o, g, w = _gated_inputs(8192, head_dim)
    z64, z32 = oracle.gated_rms_norm(o, g, w, head_dim)
    ot = torch.from_numpy(o).double().reshape(2, -1, head_dim)
    ref = (torch.nn.functional.rms_norm(ot, (head_dim,), weight=torch.from_numpy(w).double(),
                                        eps=EPS32).reshape(2, -1)
           * torch.sigmoid(torch.from_numpy(g).double())).numpy()
    assert np.all(np.abs(z64 - ref) <= 1e-14 * np.abs(ref) + 1e-300)
    assert np.array_equal(z32, z64.astype(np.float32))


def test_gated_norm_saturated_and_zero_gate():
    # g = 40: 1 + exp(-40) rounds to 1 in f64, so the gate is exactly 1 and every head is the
    # plain RMSNorm of its own 128 values (torch's rms_norm on that slice as a row).  g = 0:
    # the gate is exactly 1/2, so z is exactly half of that.
    head_dim = 128
    o, _, w = _gated_inputs(1024, head_dim)
    z_one, _ = oracle.gated_rms_norm(o, np.full_like(o, 40.0), w, head_dim)
    z_half, _ = oracle.gated_rms_norm(o, np.zeros_like(o), w, head_dim)
    assert np.array_equal(z_half, 0.5 * z_one)
    for r in range(2):
        for h in range(1024 // head_dim):
            sl = slice(h * head_dim, (h + 1) * head_dim)
            ref = torch.nn.functional.rms_norm(torch.from_numpy(o[r, sl]).double(), (head_dim,),
                                               weight=torch.from_numpy(w).double(),
                                               eps=EPS32).numpy()
            assert np.all(np.abs(z_one[r, sl] - ref) <= 1e-14 * np.abs(ref))
    # a whole-row norm would differ: the heads' mean squares are not all equal
    whole = torch.nn.functional.rms_norm(torch.from_numpy(o).double(), (1024,),
                                         weight=torch.from_numpy(np.tile(w, 8)).double(),
                                         eps=EPS32).numpy()
    assert np.max(np.abs(whole - z_one) / np.abs(whole)) > 1e-3


@pytest.mark.parametrize("c", [2.0 ** -10, 0.75, -3.5])
def test_gated_norm_constant_head_closed_form(c):
    # o = c over the head, w = 1, g = 0: z = (c / sqrt(c^2 + eps)) / 2
    head_dim = 64
    o = np.full((1, 2 * head_dim), c, dtype=np.float32)
    z64, _ = oracle.gated_rms_norm(o, np.zeros_like(o), np.ones(head_dim, np.float32), head_dim)
    getcontext().prec = 50
    dc = Decimal(c)
    want = float(dc / (dc * dc + Decimal(EPS32)).sqrt() / 2)
    assert np.all(np.abs(z64 - want) <= 4e-16 * abs(want))


def test_gated_norm_decimal_reference():
    getcontext().prec = 50
    head_dim = 128
    o, g, w = _gated_inputs(2 * head_dim, head_dim, nrows=1, seed=31)
    z64, _ = oracle.gated_rms_norm(o, g, w, head_dim)
    for h in range(2):
        sl = range(h * head_dim, (h + 1) * head_dim)
        ss = sum(Decimal(float(o[0, j])) ** 2 for j in sl)
        s = 1 / (ss / head_dim + Decimal(EPS32)).sqrt()
        for j in sl:
            gd = Decimal(float(g[0, j]))
            want = Decimal(float(o[0, j])) * Decimal(float(w[j % head_dim])) * s / (1 + (-gd).exp())
            assert abs(Decimal(float(z64[0, j])) - want) <= abs(want) * Decimal(2) ** -50, j


def test_gated_norm_heads_independent_and_gate_symmetry():
    head_dim = 128
    o, g, w = _gated_inputs(1024, head_dim)
    z64, _ = oracle.gated_rms_norm(o, g, w, head_dim)
    # changing head 3 leaves every other head's output unchanged
    o2 = o.copy()
    o2[:, 3 * head_dim:4 * head_dim] *= np.float32(3.0)
    z2, _ = oracle.gated_rms_norm(o2, g, w, head_dim)
    keep = np.ones(1024, bool)
    keep[3 * head_dim:4 * head_dim] = False
    assert np.array_equal(z2[:, keep], z64[:, keep])
    # permuting whole heads permutes the output
    perm = np.concatenate([np.arange(h * head_dim, (h + 1) * head_dim) for h in (5, 0, 7, 2, 1, 6, 4, 3)])
    zp, _ = oracle.gated_rms_norm(o[:, perm], g[:, perm], w, head_dim)
    assert np.array_equal(zp, z64[:, perm])
    # sigmoid(g) + sigmoid(-g) = 1
    zn, _ = oracle.gated_rms_norm(o, -g, w, head_dim)
    z1, _ = oracle.gated_rms_norm(o, np.full_like(g, 40.0), w, head_dim)
    assert np.allclose(z64 + zn, z1, rtol=1e-14, atol=1e-15)
