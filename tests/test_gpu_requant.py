"""GPU parity of the load-time e4m3 -> Q8_0 requantiser (gemv_e4m3_bench.rs, module doc QUESTION:
the ship path dequantises FP8 checkpoints to a Q8_0 slab at load) against the CPU oracle.
The output is bytes, so the bar is byte-for-byte equality: every fp16 scale and every int8."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, oracle_threads, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def _run(fg, W, in_f, out_f, scale=None, grid=None, q_row_bytes=None, offset=0, fill=0):
    """Requantise on the GPU into a buffer prefilled with `fill`; returns [out_f, q_row_bytes]."""
    nb = in_f // 32
    qrb = nb * 34 if q_row_bytes is None else q_row_bytes
    buf = torch.full((offset + out_f * qrb,), fill, dtype=torch.uint8, device=dev())
    Wq = buf[offset:]
    Wd = to_dev(W)
    if grid is None:
        fg.requant_e4m3_q8_0(Wd, W.shape[1], scale, Wq, qrb, in_f, out_f)
    else:
        fg.requant_e4m3_blk128_q8_0(Wd, W.shape[1], to_dev(grid), grid.shape[1], Wq, qrb, in_f,
                                    out_f)
    return host(Wq).reshape(out_f, qrb)


# Shapes [out_f, in_f]: one block up to several 256-block workgroups per row, ragged in both
# directions; in_f % 256 != 0 (96, 160, 288, 1056, 8224) takes the 2-byte store path.
SHAPES = [(1, 32), (7, 96), (130, 160), (131, 288), (257, 1056), (33, 8224), (64, 4096),
          (129, 8704), (5, 24576), (3, 65536)]


@pytest.mark.parametrize("out_f,in_f", SHAPES)
@pytest.mark.parametrize("arm", ["scale_pow2", "scale_inexact", "blk128"])
def test_requant_matches_oracle_bytes(fg, arm, out_f, in_f):
    case(f"requant {arm} out_f={out_f} in_f={in_f}")
    W = synth.e4m3_weights(out_f, in_f)
    if arm == "blk128":
        grid = synth.blk128_grid(out_f, in_f)
        got = _run(fg, W, in_f, out_f, grid=grid)
        want = oracle.requant_q8_0(W, in_f, in_f, out_f, grid=grid)
    else:
        S = 2.0 ** -4 if arm == "scale_pow2" else 0.3
        got = _run(fg, W, in_f, out_f, scale=S)
        want = oracle.requant_q8_0(W, in_f, in_f, out_f, scale=S)
    assert np.array_equal(got, want)


# The 27B-class projection shapes, every row against the oracle (rows split across host
# threads; each oracle call writes only its own rows).
@pytest.mark.parametrize("out_f,in_f", [(5120, 5120), (17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("arm", ["scale_pow2", "blk128"])
def test_requant_full_shapes_every_row(fg, arm, out_f, in_f):
    import concurrent.futures as cf
    case(f"requant full {arm} out_f={out_f} in_f={in_f}")
    W = synth.e4m3_weights(out_f, in_f)
    grid = synth.blk128_grid(out_f, in_f) if arm == "blk128" else None
    got = _run(fg, W, in_f, out_f, scale=None if grid is not None else 2.0 ** -4, grid=grid)

    def part(rows):
        if grid is not None:
            return oracle.requant_q8_0(W, in_f, in_f, out_f, grid=grid, rows=rows)
        return oracle.requant_q8_0(W, in_f, in_f, out_f, scale=2.0 ** -4, rows=rows)

    nth = oracle_threads()
    step = (out_f + nth - 1) // nth
    ranges = [(r, min(out_f, r + step)) for r in range(0, out_f, step)]
    with cf.ThreadPoolExecutor(max_workers=nth) as ex:
        parts = list(ex.map(part, ranges))
    for (r0, r1), want in zip(ranges, parts):
        assert np.array_equal(got[r0:r1], want[r0:r1]), (r0, r1)


def test_requant_padded_and_unaligned_rows_leave_padding_alone(fg):
    case("requant padded rows")
    out_f, in_f = 9, 512
    nb = in_f // 32
    W = synth.e4m3_weights(out_f, in_f)
    want = oracle.requant_q8_0(W, in_f, in_f, out_f, scale=0.5, q_row_bytes=nb * 34 + 6)
    for offset in (0, 2):  # 16-byte aligned output, then 2-byte aligned only
        got = _run(fg, W, in_f, out_f, scale=0.5, q_row_bytes=nb * 34 + 6, offset=offset,
                   fill=0xAB)
        assert np.array_equal(got[:, :nb * 34], want[:, :nb * 34])
        assert np.all(got[:, nb * 34:] == 0xAB)


# Blocks are numbered across rows (block g is block g % nb of row g / nb), so a workgroup's 256
# blocks can span many rows.  Padded input rows, packed and padded output rows, and every store
# mode: 16-byte (packed, total blocks % 8 == 0), 2-byte runs (packed otherwise, or an output
# only 2-byte aligned) and per-block stores (padded output).
@pytest.mark.parametrize("out_f,in_f,pad", [(37, 96, 16), (131, 288, 48), (65, 8704, 16),
                                            (300, 256, 32), (3, 32, 16)])
@pytest.mark.parametrize("out_pad,offset", [(0, 0), (0, 2), (4, 0)])
def test_requant_padded_input_rows_and_row_crossing_workgroups(fg, out_f, in_f, pad, out_pad,
                                                                offset):
    case(f"requant strided out_f={out_f} in_f={in_f} pad={pad} out_pad={out_pad} off={offset}")
    nb = in_f // 32
    W = synth.e4m3_weights(out_f, in_f + pad)
    grid = synth.blk128_grid(out_f, in_f)
    qrb = nb * 34 + out_pad
    for kw in ({"scale": 0.3}, {"grid": grid}):
        want = oracle.requant_q8_0(W, in_f + pad, in_f, out_f, q_row_bytes=qrb, **kw)
        got = _run(fg, W, in_f, out_f, q_row_bytes=qrb, offset=offset, fill=0xAB, **kw)
        assert np.array_equal(got[:, :nb * 34], want[:, :nb * 34]), list(kw)
        assert np.all(got[:, nb * 34:] == 0xAB)


def test_requant_launch_split_at_two_to_the_30_blocks(fg):
    """A plane of more than 2^30 blocks is requantised in row ranges of 2^30 blocks (a multiple
    of 128 rows, so the block-128 grid row of a range starts on its first tile).  in_f = 65536:
    ranges of 524288 rows; the rows on both sides of the split, and the first and last rows, are
    checked against the oracle, per 128-row tile (a row's bytes depend only on the row and on
    its tile's grid value)."""
    in_f, nb, split = 65536, 2048, 524288
    out_f = split + 200
    case(f"requant launch split out_f={out_f} in_f={in_f}")
    base = synth.e4m3_weights(256, in_f)          # row r of the plane is base row r % 256
    grid = synth.blk128_grid(out_f, in_f)
    Wd = to_dev(base).repeat((out_f + 255) // 256, 1)[:out_f]
    Wq = torch.empty((out_f, nb * 34), dtype=torch.uint8, device=dev())
    check = [0, 1, split - 2, split - 1, split, split + 1, out_f - 1]
    try:
        for arm in ("scale", "grid"):
            Wq.fill_(0xAB)
            if arm == "scale":
                fg.requant_e4m3_q8_0(Wd, in_f, 0.3, Wq, nb * 34, in_f, out_f)
            else:
                fg.requant_e4m3_blk128_q8_0(Wd, in_f, to_dev(grid), grid.shape[1], Wq, nb * 34,
                                            in_f, out_f)
            torch.cuda.synchronize()
            for r in check:
                t0 = r // 128 * 128
                tile_rows = np.stack([base[(t0 + i) % 256] for i in range(128)])
                kw = {"scale": 0.3} if arm == "scale" else {"grid": grid[t0 // 128:t0 // 128 + 1]}
                want = oracle.requant_q8_0(tile_rows, in_f, in_f, 128, rows=(r - t0, r - t0 + 1),
                                           **kw)[r - t0]
                assert np.array_equal(host(Wq[r]), want), (arm, r)
    finally:
        del Wd, Wq
        torch.cuda.empty_cache()


def test_requant_special_blocks(fg):
    case("requant special blocks")
    in_f = 256
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    rows = [
        np.resize(codes, in_f),                      # every finite code
        np.zeros(in_f, np.uint8),                    # d = 0
        np.tile(np.array([0x00, 0x80], np.uint8), in_f // 2),  # signed zeros
        np.resize(np.arange(1, 8, dtype=np.uint8), in_f),      # subnormal codes only
        np.full(in_f, 0x7E, np.uint8),               # all +448
        np.full(in_f, 0xFE, np.uint8),               # all -448
    ]
    W = np.stack(rows)
    for S in (1.0, 2.0 ** -20, 2.0 ** 10, 2.0 ** 20, 0.3):  # 2^-20: fp16 subnormal d; 2^20: inf
        got = _run(fg, W, in_f, W.shape[0], scale=S)
        want = oracle.requant_q8_0(W, in_f, in_f, W.shape[0], scale=S)
        assert np.array_equal(got, want), S


def test_gemv_over_requantised_weights(fg):
    case("requant then gemv_q8_0_q81")
    out_f, in_f = 300, 2048
    W = synth.e4m3_weights(out_f, in_f)
    grid = synth.blk128_grid(out_f, in_f)
    nb = in_f // 32
    Qd = torch.empty(out_f * nb * 34, dtype=torch.uint8, device=dev())
    fg.requant_e4m3_blk128_q8_0(to_dev(W), in_f, to_dev(grid), grid.shape[1], Qd, nb * 34, in_f,
                                out_f)
    Qo = oracle.requant_q8_0(W, in_f, in_f, out_f, grid=grid)
    x = synth.x_rows(in_f, 2)
    qs, d = oracle.quantize_q8_1(x)
    y = torch.empty(2 * out_f, device=dev())
    fg.gemv_q8_0_q81(Qd, nb * 34, to_dev(qs), to_dev(d), y, 2, in_f, out_f)
    yg = host(y).reshape(2, out_f)
    yo, A = oracle.gemv_q8_0(Qo, nb * 34, qs, d, in_f, out_f)
    assert np.all(np.abs(yg - yo) <= 1e-5 * A)
    # same bytes -> same GEMV bits
    y2 = torch.empty(2 * out_f, device=dev())
    fg.gemv_q8_0_q81(to_dev(Qo.reshape(-1)), nb * 34, to_dev(qs), to_dev(d), y2, 2, in_f, out_f)
    assert host(y2).tobytes() == yg.tobytes()


def test_requant_binding_rejects_bad_arguments(fg):
    W = torch.zeros(64, dtype=torch.uint8, device=dev())
    Wq = torch.zeros(68, dtype=torch.uint8, device=dev())
    with pytest.raises(fg.Fp8GemvError):
        fg.requant_e4m3_q8_0(W, 64, 1.0, Wq, 68, 48, 1)
    with pytest.raises(ValueError):
        fg.requant_e4m3_q8_0(W.cpu(), 64, 1.0, Wq, 68, 64, 1)
    with pytest.raises(ValueError):
        fg.requant_e4m3_q8_0(W, 64, 1.0, Wq[:60], 68, 64, 1)
