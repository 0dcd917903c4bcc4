"""Seeded random requantiser cases against the oracle, byte for byte (gemv_e4m3_bench.rs,
module doc QUESTION: the load-time e4m3 -> Q8_0 slab): in_f, out_f, the scale (a power of
two, an inexact one, or the block-128 grid), padded input strides, padded output rows and an
output offset of 2 bytes or more are drawn from a fixed-seed generator.  The output buffer is
prefilled, so the padding bytes must come back untouched."""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 160


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


@pytest.mark.parametrize("block", range(4))
def test_requant_random_cases_match_oracle(fg, block):
    rng = random.Random(0x2E0A + block)
    for i in range(N_CASES // 4):
        in_f = 32 * rng.randint(1, 2048)
        out_f = rng.randint(1, 600)
        while out_f * in_f > 2e7 and out_f > 1:
            out_f //= 2
        arm = rng.choice(["pow2", "inexact", "blk128"])
        pad_in = rng.choice([0, 0, 16, 48])
        pad_out = rng.choice([0, 0, 2, 6, 34])
        offset = rng.choice([0, 2, 16])
        nb = in_f // 32
        rb, qrb = in_f + pad_in, nb * 34 + pad_out
        W = synth.e4m3_weights(out_f, in_f)
        Wp = np.zeros((out_f, rb), np.uint8)
        Wp[:, :in_f] = W
        case(f"random requant block {block} #{i}: {arm} out_f={out_f} in_f={in_f} "
             f"row_bytes={rb} q_row_bytes={qrb} offset={offset}")
        buf = torch.full((offset + out_f * qrb,), 0xA5, dtype=torch.uint8, device=dev())
        Wq = buf[offset:]
        Wd = to_dev(Wp)
        if arm == "blk128":
            grid = synth.blk128_grid(out_f, in_f)
            fg.requant_e4m3_blk128_q8_0(Wd, rb, to_dev(grid), grid.shape[1], Wq, qrb, in_f, out_f)
            want = oracle.requant_q8_0(Wp, rb, in_f, out_f, grid=grid, q_row_bytes=qrb)
        else:
            S = 2.0 ** rng.randint(-9, 3) if arm == "pow2" else rng.uniform(0.01, 3.0)
            fg.requant_e4m3_q8_0(Wd, rb, S, Wq, qrb, in_f, out_f)
            want = oracle.requant_q8_0(Wp, rb, in_f, out_f, scale=S, q_row_bytes=qrb)
        got = host(buf)
        assert np.all(got[:offset] == 0xA5), f"case {i}: bytes before the output written"
        got = got[offset:].reshape(out_f, qrb)
        assert np.array_equal(got[:, :nb * 34], want[:, :nb * 34]), f"case {i}: blocks differ"
        assert np.all(got[:, nb * 34:] == 0xA5), f"case {i}: row padding written"
