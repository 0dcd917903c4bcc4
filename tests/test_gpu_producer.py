"""GPU parity of the producer (RMSNorm -> q8_1) against the CPU oracle, and byte identity of
the fused kernel with the two-launch chain (q8_fuse_gate.rs, module doc and `run_shape`)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import read_blocks
from gpu_util import case, dev, host, to_dev

pytestmark = pytest.mark.gpu

# The gate page's three site widths (1536, 4096, 8192), the 27B projection widths, and small,
# odd-window and maximal widths.
NCOLS = [32, 96, 1056, 1536, 2048, 4096, 5120, 8192, 17408, 65536]


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def _gpu_producer(fg, x, w, with_z=True):
    nrows, ncols = x.shape
    xd, wd = to_dev(x), to_dev(w)
    z = torch.empty((nrows, ncols), device=dev()) if with_z else None
    qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((nrows, ncols // 32), device=dev())
    fg.rmsnorm_q8_1(xd, wd, z, qs, d, ncols, nrows)
    return (host(z) if with_z else None), host(qs), host(d)


def _gpu_chain(fg, x, w):
    nrows, ncols = x.shape
    xd, wd = to_dev(x), to_dev(w)
    z = torch.empty((nrows, ncols), device=dev())
    qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((nrows, ncols // 32), device=dev())
    fg.rms_norm_f32(xd, wd, z, ncols, nrows)
    fg.quantize_q8_1(z, qs, d, nrows, ncols)
    return host(z), host(qs), host(d)


@pytest.mark.parametrize("nrows", [1, 3])
@pytest.mark.parametrize("ncols", NCOLS)
def test_rmsnorm_q8_1_matches_oracle(fg, ncols, nrows):
    case(f"rmsnorm_q8_1 ncols={ncols} nrows={nrows}")
    x = synth.x_rows(ncols, nrows)
    w = synth.gain(ncols)
    z, qs, d = _gpu_producer(fg, x, w)
    ref = oracle.rmsnorm_q8_1(x, w)
    z64, d64 = ref["z64"], ref["d64"]
    # required bars: z and d within 1e-5 relative, qs bit-exact on the GPU's own z
    assert np.all(np.abs(z - z64) <= 1e-5 * np.abs(z64))
    assert np.all(np.abs(d - d64) <= 1e-5 * d64)
    q_o, d_o = oracle.quantize_q8_1(z)
    assert np.array_equal(qs, q_o) and np.array_equal(d.view(np.uint32), d_o.view(np.uint32))
    # this design computes z with the oracle's own f64 sequence, so z, qs and d agree bitwise
    assert np.array_equal(z.view(np.uint32), ref["z32"].view(np.uint32))
    assert np.array_equal(qs, ref["qs"]) and np.array_equal(d, ref["d"])


def test_max_nrows(fg):
    # the largest row count the library accepts (the launch grid's y dimension indexes rows)
    nrows, ncols = 65535, 64
    case(f"rmsnorm_q8_1 ncols={ncols} nrows={nrows}")
    x = synth.x_rows(ncols, nrows)
    w = synth.gain(ncols)
    z, qs, d = _gpu_producer(fg, x, w)
    ref = oracle.rmsnorm_q8_1(x, w)
    assert np.array_equal(z.view(np.uint32), ref["z32"].view(np.uint32))
    assert np.array_equal(qs, ref["qs"]) and np.array_equal(d, ref["d"])
    zc, qc, dc = _gpu_chain(fg, x, w)
    assert zc.tobytes() == z.tobytes() and qc.tobytes() == qs.tobytes() and dc.tobytes() == d.tobytes()


@pytest.mark.parametrize("nrows", [1, 2])
@pytest.mark.parametrize("ncols", [1536, 4096, 8192, 32, 5120, 17408])
def test_fused_is_byte_identical_to_chain(fg, ncols, nrows):
    case(f"fused vs chain ncols={ncols} nrows={nrows}")
    x = synth.x_rows(ncols, nrows)
    w = synth.gain(ncols)
    zf, qf, df = _gpu_producer(fg, x, w)
    zc, qc, dc = _gpu_chain(fg, x, w)
    assert zf.tobytes() == zc.tobytes()
    assert qf.tobytes() == qc.tobytes()
    assert df.tobytes() == dc.tobytes()
    _, qn, dn = _gpu_producer(fg, x, w, with_z=False)   # z = NULL skips only the z store
    assert qn.tobytes() == qf.tobytes() and dn.tobytes() == df.tobytes()


@pytest.mark.parametrize("ncols,nrows", [(32, 1), (5120, 1), (17408, 1), (4096, 8), (2080, 3)])
def test_quantize_q8_1_of_raw_x_matches_oracle(fg, ncols, nrows):
    case(f"quantize_q8_1 ncols={ncols} nrows={nrows}")
    x = synth.x_rows(ncols, nrows)
    qs = torch.empty((nrows, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((nrows, ncols // 32), device=dev())
    fg.quantize_q8_1(to_dev(x), qs, d, nrows, ncols)
    q_o, d_o = oracle.quantize_q8_1(x)
    assert np.array_equal(host(qs), q_o)
    assert np.array_equal(host(d).view(np.uint32), d_o.view(np.uint32))


def test_quantize_golden_blocks(fg):
    case("quantize_q8_1 golden blocks")
    blocks = read_blocks("q8_1_blocks.txt")
    z = np.array([b["z"] for b in blocks.values()], dtype=np.float32).reshape(1, -1)
    ncols = z.shape[1]
    qs = torch.empty((1, ncols), dtype=torch.int8, device=dev())
    d = torch.empty((1, ncols // 32), device=dev())
    fg.quantize_q8_1(to_dev(z), qs, d, 1, ncols)
    qh, dh = host(qs).reshape(-1, 32), host(d).reshape(-1)
    for i, (name, b) in enumerate(blocks.items()):
        assert qh[i].tolist() == b["q"], name
        if "d" in b:
            assert float(dh[i]) == b["d"], name


def test_producer_special_rows(fg):
    # a zero row (s = 1/sqrt(eps), z = 0, d = 0, q = 0), a row with one all-zero block, a row
    # of huge values, a row of tiny values where eps dominates
    case("rmsnorm_q8_1 special rows")
    ncols = 256
    x = synth.x_rows(ncols, 4)
    x[0] = 0
    x[1, 32:64] = 0
    x[2] *= np.float32(1e30)
    x[3] *= np.float32(2.0 ** -20)
    w = synth.gain(ncols)
    z, qs, d = _gpu_producer(fg, x, w)
    ref = oracle.rmsnorm_q8_1(x, w)
    assert np.array_equal(z.view(np.uint32), ref["z32"].view(np.uint32))
    assert np.array_equal(qs, ref["qs"]) and np.array_equal(d, ref["d"])
    assert np.all(qs[0] == 0) and np.all(d[0] == 0) and np.all(qs[1, 32:64] == 0) and d[1, 1] == 0
