"""Seeded random producer cases (q8_fuse_gate.rs, module doc and `run_shape`): ncols, nrows
and the input rows (seeded xorshift draws, some rows scaled by powers of two to spread their
magnitudes) are drawn from a fixed-seed generator.  The fused producer's z, qs and d must equal
the oracle's bit for bit, and the two-launch chain must give the same bytes."""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 120


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


@pytest.mark.parametrize("block", range(4))
def test_rmsnorm_q8_1_random_cases_match_oracle_and_chain(fg, block):
    rng = random.Random(0x9A0D + block)
    for i in range(N_CASES // 4):
        ncols = 32 * rng.randint(1, 2048)
        nrows = rng.randint(1, 6)
        seed = rng.randint(1, 10 ** 6)
        x = np.stack([synth.f32(seed + r, ncols) * np.float32(2.0 ** rng.randint(-20, 20))
                      for r in range(nrows)]).astype(np.float32)
        w = synth.f32(seed ^ 0x77, ncols)
        case(f"random producer block {block} #{i}: ncols={ncols} nrows={nrows}")
        xd, wd = to_dev(x), to_dev(w)
        z = torch.empty((nrows, ncols), device=dev())
        qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
        d = torch.empty((nrows, ncols // 32), device=dev())
        fg.rmsnorm_q8_1(xd, wd, z, qs, d, ncols, nrows)
        zc = torch.empty_like(z)
        qc = torch.empty_like(qs)
        dc = torch.empty_like(d)
        fg.rms_norm_f32(xd, wd, zc, ncols, nrows)
        fg.quantize_q8_1(zc, qc, dc, nrows, ncols)
        z, qs, d, zc, qc, dc = (host(t) for t in (z, qs, d, zc, qc, dc))
        ref = oracle.rmsnorm_q8_1(x, w)
        assert np.array_equal(z.view(np.uint32), ref["z32"].view(np.uint32)), f"case {i}: z"
        assert np.array_equal(qs, ref["qs"]) and np.array_equal(d, ref["d"]), f"case {i}: q8_1"
        assert zc.tobytes() == z.tobytes() and qc.tobytes() == qs.tobytes() and \
            dc.tobytes() == d.tobytes(), f"case {i}: chain differs from fused"
