"""GPU parity of the KDA gated-norm producer (q8_fuse_gate.rs, module doc and `main`: the KDA
qkv width 64 heads x 128 head_dim = 8192 is the KDA gated-norm site) against the CPU oracle:
per head RMSNorm x gain x sigmoid(gate), then q8_1; and byte identity of the fused kernel with
the two-launch chain gated_rms_norm_f32 -> quantize_q8_1."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def _inputs(ncols, head_dim, nrows):
    o = np.stack([synth.f32(0x0DA0 ^ ncols ^ (t << 20), ncols) for t in range(nrows)])
    g = np.stack([synth.f32(0x6A7E ^ ncols ^ (t << 20), ncols) for t in range(nrows)])
    return o, g, synth.gain(head_dim)


def _assert_z_matches(z, z64):
    """z equals the oracle's rounding of z64, except where z64 sits so close to an f32 rounding
    midpoint that the device and host exp (each within an ulp of f64) may decide differently;
    there z may be the other neighbour."""
    z32 = z64.astype(np.float32)
    diff = z.view(np.uint32) != z32.view(np.uint32)
    if diff.any():
        a, b = z[diff].astype(np.float64), z32[diff].astype(np.float64)
        mid = (a + b) / 2
        near = np.abs(z64[diff] - mid) <= np.abs(mid) * 2.0 ** -45
        adjacent = np.abs(z[diff].view(np.int32) - z32[diff].view(np.int32)) == 1
        assert np.all(near & adjacent), f"{diff.sum()} values off"


def _gpu(fg, o, g, w, head_dim, fused=True, with_z=True):
    nrows, ncols = o.shape
    od, gd, wd = to_dev(o), to_dev(g), to_dev(w)
    z = torch.empty((nrows, ncols), device=dev()) if with_z else None
    qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((nrows, ncols // 32), device=dev())
    if fused:
        fg.gated_rmsnorm_q8_1(od, gd, wd, z, qs, d, ncols, head_dim, nrows, EPS)
    else:
        fg.gated_rms_norm_f32(od, gd, wd, z, ncols, head_dim, nrows, EPS)
        fg.quantize_q8_1(z, qs, d, nrows, ncols)
    return (host(z) if with_z else None), host(qs), host(d)


# 8192 = 64 heads x 128 is the page's KDA width; the rest cover one head up to the largest row,
# rows that end inside a 1024-column workgroup, and every supported head_dim.
CASES = [(128, 128), (8192, 128), (1152, 128), (96, 32), (8192, 32), (4160, 64), (8192, 64),
         (256, 256), (8448, 256), (65536, 128)]


@pytest.mark.parametrize("nrows", [1, 3])
@pytest.mark.parametrize("ncols,head_dim", CASES)
def test_gated_rmsnorm_q8_1_matches_oracle_and_chain(fg, ncols, head_dim, nrows):
    case(f"gated_rmsnorm_q8_1 ncols={ncols} head_dim={head_dim} nrows={nrows}")
    o, g, w = _inputs(ncols, head_dim, nrows)
    z, qs, d = _gpu(fg, o, g, w, head_dim)
    z64, _ = oracle.gated_rms_norm(o, g, w, head_dim, EPS)
    _assert_z_matches(z, z64)
    # the q8_1 step on the GPU's own z is bit-exact
    q_o, d_o = oracle.quantize_q8_1(z)
    assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
    # fused == chain, byte for byte; z = NULL changes nothing else
    zc, qc, dc = _gpu(fg, o, g, w, head_dim, fused=False)
    assert zc.tobytes() == z.tobytes() and qc.tobytes() == qs.tobytes()
    assert dc.tobytes() == d.tobytes()
    _, qn, dn = _gpu(fg, o, g, w, head_dim, with_z=False)
    assert qn.tobytes() == qs.tobytes() and dn.tobytes() == d.tobytes()


def test_gated_special_values(fg):
    # saturated gates (100, +-1e30), a nearly closed gate (-30: z ~ 1e-13 stays a normal f32,
    # so every block has a finite 1/d), a zero gate, a zero head (d = 0 blocks) and a head of
    # tiny values
    case("gated_rmsnorm_q8_1 special values")
    head_dim, ncols = 128, 1024
    o, g, w = _inputs(ncols, head_dim, 1)
    g[0, :128] = 100.0
    g[0, 128:256] = -30.0
    g[0, 256:384] = 0.0
    g[0, 384:512:2] = 1e30
    g[0, 385:512:2] = -1e30
    o[0, 512:640] = 0.0
    o[0, 640:768] = np.float32(1e-20)
    z, qs, d = _gpu(fg, o, g, w, head_dim)
    z64, _ = oracle.gated_rms_norm(o, g, w, head_dim, EPS)
    _assert_z_matches(z, z64)
    q_o, d_o = oracle.quantize_q8_1(z)
    assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
    assert np.all(d[0, 16:20] == 0) and np.all(qs[0, 512:640] == 0)


def test_gated_rejects_bad_head_dim(fg):
    # buffers large enough for every size tried, so that the library (not the binding's size
    # check) is what refuses the head_dim
    o = torch.zeros(1024, device=dev())
    qs = torch.zeros(1024, dtype=torch.int8, device=dev())
    d = torch.zeros(32, device=dev())
    for hd, ncols in ((48, 192), (512, 512), (128, 192)):
        with pytest.raises(fg.Fp8GemvError):
            fg.gated_rmsnorm_q8_1(o, o, o, None, qs, d, ncols, hd, 1)
