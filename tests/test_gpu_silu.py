"""GPU parity of the SiLU-gated producer silu(gate) * up -> q8_1 (q8_fuse_gate.rs `main`: the
MoE expert-ff activation site) against the CPU oracle, and byte identity of the fused kernel
with the two-launch chain silu_mul_f32 -> quantize_q8_1."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, to_dev

pytestmark = pytest.mark.gpu

# 1536 is the page's expert-ff width; the rest span one block to the largest row.
NCOLS = [32, 96, 1536, 4096, 8192, 65536]


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def _inputs(ncols, nrows):
    gate = np.stack([synth.f32(0xA5A5 ^ ncols ^ (t << 20), ncols) for t in range(nrows)])
    up = np.stack([synth.f32(0x5A5A ^ ncols ^ (t << 20), ncols) for t in range(nrows)])
    return gate, up


def _assert_h_matches(h, h64):
    """h equals the oracle's rounding of h64, except where h64 sits so close to an f32
    rounding midpoint that the device and host exp (each within an ulp of f64) may decide
    differently; there h may be the other neighbour."""
    h32 = h64.astype(np.float32)
    diff = h.view(np.uint32) != h32.view(np.uint32)
    if diff.any():
        a, b = h[diff].astype(np.float64), h32[diff].astype(np.float64)
        mid = (a + b) / 2
        near = np.abs(h64[diff] - mid) <= np.abs(mid) * 2.0 ** -45
        adjacent = np.abs(h[diff].view(np.int32) - h32[diff].view(np.int32)) == 1
        assert np.all(near & adjacent), f"{diff.sum()} values off"


def _gpu(fg, gate, up, fused=True, with_h=True):
    nrows, ncols = gate.shape
    gd, ud = to_dev(gate), to_dev(up)
    h = torch.empty((nrows, ncols), device=dev()) if with_h else None
    qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((nrows, ncols // 32), device=dev())
    if fused:
        fg.silu_mul_q8_1(gd, ud, h, qs, d, ncols, nrows)
    else:
        fg.silu_mul_f32(gd, ud, h, ncols, nrows)
        fg.quantize_q8_1(h, qs, d, nrows, ncols)
    return (host(h) if with_h else None), host(qs), host(d)


@pytest.mark.parametrize("nrows", [1, 3])
@pytest.mark.parametrize("ncols", NCOLS)
def test_silu_mul_q8_1_matches_oracle_and_chain(fg, ncols, nrows):
    case(f"silu_mul_q8_1 ncols={ncols} nrows={nrows}")
    gate, up = _inputs(ncols, nrows)
    h, qs, d = _gpu(fg, gate, up)
    h64, _ = oracle.silu_mul(gate, up)
    _assert_h_matches(h, h64)
    q_o, d_o = oracle.quantize_q8_1(h)
    assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
    hc, qc, dc = _gpu(fg, gate, up, fused=False)
    assert hc.tobytes() == h.tobytes() and qc.tobytes() == qs.tobytes()
    assert dc.tobytes() == d.tobytes()
    _, qn, dn = _gpu(fg, gate, up, with_h=False)
    assert qn.tobytes() == qs.tobytes() and dn.tobytes() == d.tobytes()


def test_silu_mul_special_values(fg):
    case("silu_mul special values")
    g = np.array([0.0, -0.0, 100.0, -100.0, 1e30, -1e30, 88.0, -88.0, 1e-30, -1e-30, 20.0,
                  -20.0, 3.0, -3.0, 0.5, -0.5] * 4, dtype=np.float32)[None, :]
    u = np.array([1.0, 1.0, 2.0, 2.0, 1.0, 1.0, -1.0, -1.0, 1e30, 1e30, 0.0, -0.0, 1e-3,
                  -1e-3, 4.0, 4.0] * 4, dtype=np.float32)[None, :]
    h, qs, d = _gpu(fg, g, u)
    h64, _ = oracle.silu_mul(g, u)
    _assert_h_matches(h, h64)
    q_o, d_o = oracle.quantize_q8_1(h)
    assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
