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


@pytest.mark.parametrize("block", range(2))
def test_silu_and_gated_random_cases_match_oracle_and_chain(fg, block):
    """The SiLU-gated and KDA gated-norm producers on random widths, head sizes, row counts and
    gate magnitudes.  z (or h) equals the oracle's f32 rounding except within 2^-45 of an f32
    midpoint, where the device and host exp may round apart; qs and d are bit-exact on the
    device's own z; chain == fused, byte for byte."""
    from test_gpu_gated import _assert_z_matches
    rng = random.Random(0x51E0 + block)
    for i in range(20):
        nrows = rng.randint(1, 4)
        seed = rng.randint(1, 10 ** 6)
        gscale = np.float32(2.0 ** rng.randint(-3, 5))
        if rng.random() < 0.5:
            ncols = 32 * rng.randint(1, 2048)
            g = np.stack([synth.f32(seed + r, ncols) * gscale for r in range(nrows)])
            u = np.stack([synth.f32((seed ^ 0x55) + r, ncols) for r in range(nrows)])
            g, u = g.astype(np.float32), u.astype(np.float32)
            case(f"random silu block {block} #{i}: ncols={ncols} nrows={nrows}")
            gd, ud = to_dev(g), to_dev(u)
            outs = []
            for fused in (True, False):
                h = torch.empty((nrows, ncols), device=dev())
                qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
                d = torch.empty((nrows, ncols // 32), device=dev())
                if fused:
                    fg.silu_mul_q8_1(gd, ud, h, qs, d, ncols, nrows)
                else:
                    fg.silu_mul_f32(gd, ud, h, ncols, nrows)
                    fg.quantize_q8_1(h, qs, d, nrows, ncols)
                outs.append((host(h), host(qs), host(d)))
            h64, _ = oracle.silu_mul(g, u)
        else:
            head_dim = rng.choice([32, 64, 128, 256])
            ncols = head_dim * rng.randint(1, 65536 // head_dim)
            while ncols * nrows > 300000 and ncols > head_dim:
                ncols = (ncols // 2 // head_dim) * head_dim or head_dim
            o = np.stack([synth.f32(seed + r, ncols) for r in range(nrows)]).astype(np.float32)
            g = np.stack([synth.f32((seed ^ 0x77) + r, ncols) * gscale
                          for r in range(nrows)]).astype(np.float32)
            w = synth.f32(seed ^ 0x99, head_dim)
            case(f"random gated block {block} #{i}: ncols={ncols} head_dim={head_dim} "
                 f"nrows={nrows}")
            od, gd, wd = to_dev(o), to_dev(g), to_dev(w)
            outs = []
            for fused in (True, False):
                z = torch.empty((nrows, ncols), device=dev())
                qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
                d = torch.empty((nrows, ncols // 32), device=dev())
                if fused:
                    fg.gated_rmsnorm_q8_1(od, gd, wd, z, qs, d, ncols, head_dim, nrows, 1e-6)
                else:
                    fg.gated_rms_norm_f32(od, gd, wd, z, ncols, head_dim, nrows, 1e-6)
                    fg.quantize_q8_1(z, qs, d, nrows, ncols)
                outs.append((host(z), host(qs), host(d)))
            h64, _ = oracle.gated_rms_norm(o, g, w, head_dim, 1e-6)
        (z, qs, d), (zc, qc, dc) = outs
        _assert_z_matches(z, h64)
        q_o, d_o = oracle.quantize_q8_1(z)
        assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
        assert zc.tobytes() == z.tobytes() and qc.tobytes() == qs.tobytes() and \
            dc.tobytes() == d.tobytes(), f"case {i}: chain differs from fused"
