"""Seeded random GEMV cases against the oracle (gemv_e4m3_bench.rs: THE COMPARISON, THE
BLOCK-128 ARM; WHAT MADE THIS A BOUNDED WRITE for the per-row identity): container, in_f (on
and off the 256-column Q8_0 fast path), out_f, m, padded row strides and the plain or
matrix-core entry point are drawn from a fixed-seed generator, so the cases are the same on
every run.  Each output is held to |y - y_oracle| <= 1e-5 * sum |terms|; for the plain entry
points one row of each m > 1 call must also equal an m = 1 call on that row, bit for bit."""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, oracle_all_rows, to_dev

pytestmark = pytest.mark.gpu

SCALE = 2.0 ** -4
N_CASES = 240


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def _draw(rng):
    kind = rng.choice(["q8_0", "e4m3", "blk128"])
    in_f = 256 * rng.randint(1, 80) if rng.random() < 0.5 else 32 * rng.randint(1, 640)
    m = rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 20])
    out_f = rng.randint(1, 700)
    while out_f * in_f * m > 6e7 and out_f > 1:
        out_f //= 2
    mc = rng.random() < 0.5
    pad = 0
    if rng.random() < 0.3:
        pad = rng.choice([2, 16, 34, 48, 256]) if kind == "q8_0" else rng.choice([16, 32, 256])
    return kind, in_f, m, out_f, mc, pad, rng.randint(1, 10 ** 6)


def _call(fg, kind, mc, Wd, rb, gd, gcols, qd, dd, y, m, in_f, out_f):
    sfx = "_mc" if mc else ""
    if kind == "q8_0":
        getattr(fg, "gemv_q8_0_q81" + sfx)(Wd, rb, qd, dd, y, m, in_f, out_f)
    elif kind == "e4m3":
        getattr(fg, "gemv_e4m3_q81" + sfx)(Wd, rb, SCALE, qd, dd, y, m, in_f, out_f)
    else:
        getattr(fg, "gemv_e4m3_blk128_q81" + sfx)(Wd, rb, gd, gcols, qd, dd, y, m, in_f, out_f)


@pytest.mark.parametrize("block", range(4))
def test_gemv_random_cases_match_oracle(fg, block):
    rng = random.Random(0x5EED + block)
    for i in range(N_CASES // 4):
        kind, in_f, m, out_f, mc, pad, seed = _draw(rng)
        W = synth.q8_0_weights(out_f, in_f) if kind == "q8_0" else synth.e4m3_weights(out_f, in_f)
        rb0 = W.shape[1]
        rb = rb0 + pad
        Wp = np.zeros((out_f, rb), np.uint8)
        Wp[:, :rb0] = W
        grid = synth.blk128_grid(out_f, in_f) if kind == "blk128" else None
        x = np.stack([synth.f32(seed + t, in_f) for t in range(m)])
        qs, d = oracle.quantize_q8_1(x)
        case(f"random block {block} #{i}: {kind} mc={mc} out_f={out_f} in_f={in_f} m={m} "
             f"row_bytes={rb}")
        Wd, qd, dd = to_dev(Wp), to_dev(qs), to_dev(d)
        gd = to_dev(grid) if grid is not None else None
        gcols = grid.shape[1] if grid is not None else 0
        y = torch.full((m, out_f), float("nan"), device=dev())
        _call(fg, kind, mc, Wd, rb, gd, gcols, qd, dd, y, m, in_f, out_f)
        yg = host(y)
        if kind == "q8_0":
            fn = lambda rows: oracle.gemv_q8_0(Wp, rb, qs, d, in_f, out_f, rows)
        elif kind == "e4m3":
            fn = lambda rows: oracle.gemv_e4m3(Wp, rb, SCALE, qs, d, in_f, out_f, rows)
        else:
            fn = lambda rows: oracle.gemv_e4m3_blk128(Wp, rb, grid, qs, d, in_f, out_f, rows)
        yo, A = oracle_all_rows(fn, out_f)
        err = np.abs(yg.astype(np.float64) - yo)
        assert np.all(err <= 1e-5 * A), f"case {i}: {int((~(err <= 1e-5 * A)).sum())} outputs off"
        if not mc and m > 1:
            t = rng.randrange(m)
            y1 = torch.full((1, out_f), float("nan"), device=dev())
            _call(fg, kind, False, Wd, rb, gd, gcols, to_dev(qs[t:t + 1]), to_dev(d[t:t + 1]),
                  y1, 1, in_f, out_f)
            assert np.array_equal(host(y1)[0].view(np.uint32), yg[t].view(np.uint32)), \
                f"case {i}: row {t} differs from its m = 1 call"
