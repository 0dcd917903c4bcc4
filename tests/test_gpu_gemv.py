"""GPU parity of the three GEMVs (gemv_e4m3_bench.rs: THE COMPARISON, THE BLOCK-128 ARM)
against the CPU oracle: |y_gpu - y| <= 1e-5 * sum_k |term_k| per output, on the same seeded
inputs, from one-tile shapes with ragged tails up to the 27B-class projection shapes run in
the launch configuration the bench times."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, dev, host, oracle_all_rows, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
KINDS = ["q8_0", "e4m3", "blk128"]
SCALE = 2.0 ** -4  # the per-tensor scale of the e4m3 configs


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


class Case:
    """Weights of one container plus a q8_1 activation, on host and device."""

    def __init__(self, kind, out_f, in_f, m, seed=0):
        self.kind, self.out_f, self.in_f, self.m = kind, out_f, in_f, m
        if kind == "q8_0":
            self.W = synth.q8_0_weights(out_f, in_f)
        else:
            self.W = synth.e4m3_weights(out_f, in_f)
        self.row_bytes = self.W.shape[1]
        self.grid = synth.blk128_grid(out_f, in_f) if kind == "blk128" else None
        x = synth.x_rows(in_f, m)
        if seed:
            x = np.stack([synth.f32(seed + t, in_f) for t in range(m)])
        self.qs, self.d = oracle.quantize_q8_1(x)
        self.Wd = to_dev(self.W)
        self.gd = to_dev(self.grid) if self.grid is not None else None

    def gpu(self, fg, qs=None, d=None, m=None, Wd=None, row_bytes=None, mc=False):
        """The plain entry point, or with mc the matrix-core one (*_mc)."""
        m = self.m if m is None else m
        sfx = "_mc" if mc else ""
        qs = to_dev(self.qs) if qs is None else qs
        d = to_dev(self.d) if d is None else d
        Wd = self.Wd if Wd is None else Wd
        rb = self.row_bytes if row_bytes is None else row_bytes
        y = torch.full((m, self.out_f), float("nan"), device=dev())
        if self.kind == "q8_0":
            getattr(fg, "gemv_q8_0_q81" + sfx)(Wd, rb, qs, d, y, m, self.in_f, self.out_f)
        elif self.kind == "e4m3":
            getattr(fg, "gemv_e4m3_q81" + sfx)(Wd, rb, SCALE, qs, d, y, m, self.in_f, self.out_f)
        else:
            getattr(fg, "gemv_e4m3_blk128_q81" + sfx)(Wd, rb, self.gd, self.grid.shape[1], qs, d,
                                                      y, m, self.in_f, self.out_f)
        return host(y)

    def oracle_all(self):
        """The oracle over every output row, rows split across host threads."""
        return oracle_all_rows(lambda rows: self.oracle(rows), self.out_f)

    def oracle(self, rows=None):
        if self.kind == "q8_0":
            return oracle.gemv_q8_0(self.W, self.row_bytes, self.qs, self.d, self.in_f,
                                    self.out_f, rows)
        if self.kind == "e4m3":
            return oracle.gemv_e4m3(self.W, self.row_bytes, SCALE, self.qs, self.d, self.in_f,
                                    self.out_f, rows)
        return oracle.gemv_e4m3_blk128(self.W, self.row_bytes, self.grid, self.qs, self.d,
                                       self.in_f, self.out_f, rows)


def _assert_close(y, yo, A, rows=None):
    if rows is not None:
        y, yo, A = y[:, rows[0]:rows[1]], yo[:, rows[0]:rows[1]], A[:, rows[0]:rows[1]]
    err = np.abs(y.astype(np.float64) - yo)
    bad = ~(err <= TOL * A)
    assert not bad.any(), f"{bad.sum()} outputs off; worst rel {np.max(err / A):.3e}"


# Shapes [out_f, in_f] from a single window to several, with ragged tails in both directions
# (in_f not a multiple of the 1 KiB window or of 256, out_f not a multiple of the 8 rows per
# workgroup or of the 128-row grid tile).
# Beyond in_f = 8192 two waves share a row, the second starting mid-row: 8704 and 24576 split
# rows of an odd number of windows (Q8_0: 12 and 32 groups of 8 blocks, in windows of three
# groups, the last one partial), 8224 leaves a 32-column last e4m3 window, 9600 is not a
# multiple of 256 (Q8_0 generic path), 24576 is the largest in_f of that launch shape.
# More Q8_0 row lengths (in groups of 8 blocks): 9, 10, 12, 48 and 95 groups (last windows of
# 0, 1 or 2 groups past whole windows of three), single rows at the bench's in_f values, and
# out_f values that leave the last workgroup partly empty.
SMALL = [(1, 32), (7, 96), (130, 160), (131, 288), (257, 1056), (300, 2080), (64, 4096),
         (129, 4352), (33, 1280), (250, 2048), (37, 8704), (5, 8224), (131, 9600), (9, 24576),
         (13, 2304), (21, 2560), (43, 3072), (7, 12288), (11, 24320), (1, 5120), (3, 17408)]


@pytest.mark.parametrize("m", [1, 3, 5])
@pytest.mark.parametrize("out_f,in_f", SMALL)
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_small_shapes_match_oracle(fg, kind, out_f, in_f, m):
    case(f"{kind} out_f={out_f} in_f={in_f} m={m}")
    c = Case(kind, out_f, in_f, m)
    y = c.gpu(fg)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


# The 27B-class projection shapes of the bench, m = 1, the same launch as bench.py; every
# output against the oracle (run over all rows, split across host threads).
FULL = [(5120, 5120), (17408, 5120), (5120, 17408)]


@pytest.mark.parametrize("out_f,in_f", FULL)
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_full_shapes_every_row(fg, kind, out_f, in_f):
    case(f"{kind} full out_f={out_f} in_f={in_f}")
    c = Case(kind, out_f, in_f, 1)
    y = c.gpu(fg)
    assert np.all(np.isfinite(y))
    yo, A = c.oracle_all()
    _assert_close(y, yo, A)


# The projection shapes of the 27B and 1.7B sheets not covered above ([out_f, in_f]), every
# output.
SHEET = [(12288, 5120), (1024, 5120), (5120, 6144), (2048, 2048), (1024, 2048), (6144, 2048),
         (2048, 6144)]


@pytest.mark.parametrize("out_f,in_f", SHEET)
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_sheet_shapes_every_row(fg, kind, out_f, in_f):
    case(f"{kind} sheet out_f={out_f} in_f={in_f}")
    c = Case(kind, out_f, in_f, 1)
    y = c.gpu(fg)
    assert np.all(np.isfinite(y))
    yo, A = c.oracle_all()
    _assert_close(y, yo, A)


def row_reference(fg, c, t, mc=False):
    """Row t of activation rows qs/d computed alone.  Plain entry point: an m = 1 call (the
    batched arms' bit-parity gate).  Matrix cores: a 5-row call holding row t first and four
    other rows after it, so row t sits at another position among other rows."""
    if not mc:
        return c.gpu(fg, qs=to_dev(c.qs[t:t + 1]), d=to_dev(c.d[t:t + 1]), m=1)[0]
    idx = [t] + [(t + k) % c.m for k in range(1, 5)]
    return c.gpu(fg, qs=to_dev(c.qs[idx]), d=to_dev(c.d[idx]), m=5, mc=True)[0]


# m > 1 shares each weight pass between up to 8 activation rows (fewer beyond in_f = 8192);
# m = 3, 5 and 11 leave rows of the last weight pass unused, 11 takes two passes.  Each row
# of an m-row call is bit-identical to an m = 1 call on that row.
@pytest.mark.parametrize("out_f,in_f", [(17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_m_rows_bit_identical_per_row(fg, kind, out_f, in_f):
    c = Case(kind, out_f, in_f, 11)
    for m in (1, 2, 3, 4, 5, 8, 11):
        case(f"{kind} m={m} out_f={out_f} in_f={in_f}")
        y = c.gpu(fg, qs=to_dev(c.qs[:m]), d=to_dev(c.d[:m]), m=m)
        for t in range(m):
            y1 = row_reference(fg, c, t)
            assert y[t].tobytes() == y1.tobytes(), (m, t)
    # the last call (m = 11, two weight passes) against the oracle at every output
    yo, A = c.oracle_all()
    _assert_close(y, yo, A)


# The matrix-core entry points at the same shapes: each row of an m-row call is bit-identical
# to that row at another position among other rows, and every output of the last call is
# within the parity bar of the oracle.
@pytest.mark.parametrize("out_f,in_f", [(17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_matrix_core_rows_bit_identical_across_calls(fg, kind, out_f, in_f):
    c = Case(kind, out_f, in_f, 11)
    for m in (1, 2, 3, 4, 5, 8, 11):
        case(f"{kind} matrix cores m={m} out_f={out_f} in_f={in_f}")
        y = c.gpu(fg, qs=to_dev(c.qs[:m]), d=to_dev(c.d[:m]), m=m, mc=True)
        for t in range(m):
            assert y[t].tobytes() == row_reference(fg, c, t, mc=True).tobytes(), (m, t)
    yo, A = c.oracle_all()
    _assert_close(y, yo, A)


# The matrix-core kernel at its edges: in_f not a multiple of its 256-column step or of the
# 1 KiB span of the 4 waves that share a row group (so some waves have no columns), rows
# from one step to 65536 columns, out_f not a multiple of a wave's 16 rows, block-128 grids
# with several row tiles, m = 1 and 2 (most of the 8 columns empty), 3, 8 (one full pass), 9
# and 17 (a last pass of one row), 16 (two full passes).  Rows of more than 8192 columns take
# the 8-way column split.
MFMA_SHAPES = [(1, 32), (17, 288), (100, 1056), (200, 4128), (129, 8160), (65, 8192),
               (33, 8224), (300, 5120), (40, 17408), (9, 65536)]


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 16, 17])
@pytest.mark.parametrize("out_f,in_f", MFMA_SHAPES)
@pytest.mark.parametrize("kind", ["e4m3", "blk128"])
def test_gemv_matrix_core_shapes_match_oracle(fg, kind, out_f, in_f, m):
    case(f"{kind} matrix cores out_f={out_f} in_f={in_f} m={m}")
    c = Case(kind, out_f, in_f, m)
    y = c.gpu(fg, mc=True)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


# The Q8_0 matrix-core kernel (fast-path rows: in_f a multiple of the 8-block group): one
# group up to 65536 columns, groups that do not divide evenly between the waves of a row
# group (1280 = 5 groups over 4 waves, 4352 = 17, 8448 = 33 over 8), out_f not a multiple of
# 16, rows past 8192 columns split 8 ways.
Q8_MFMA_SHAPES = [(1, 256), (17, 512), (100, 1280), (200, 4352), (65, 8192), (33, 8448),
                  (300, 5120), (40, 17408), (9, 65536)]


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 16, 17])
@pytest.mark.parametrize("out_f,in_f", Q8_MFMA_SHAPES)
def test_gemv_q8_0_matrix_core_shapes_match_oracle(fg, out_f, in_f, m):
    case(f"q8_0 matrix cores out_f={out_f} in_f={in_f} m={m}")
    c = Case("q8_0", out_f, in_f, m)
    y = c.gpu(fg, mc=True)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


# Beyond the matrix-core kernels' limit (a row stride of 64 MiB or more, where 16 rows'
# offsets would leave 32 bits) the *_mc entry points run the vector kernels, bit-identical to
# m=1.
@pytest.mark.parametrize("kind", KINDS)
def test_gemv_vector_path_beyond_the_matrix_core_limits(fg, kind):
    case(f"{kind} m=8 with a 64 MiB row stride")
    out_f, in_f, m = 3, 256, 8
    c = Case(kind, out_f, in_f, m)
    rb = (1 << 26) + 16
    nbytes = c.W.shape[1]
    flat = torch.zeros((out_f - 1) * rb + nbytes, dtype=torch.uint8, device=dev())
    for r in range(out_f):
        flat[r * rb:r * rb + nbytes] = torch.from_numpy(c.W[r]).to(dev())
    y = c.gpu(fg, Wd=flat, row_bytes=rb, mc=True)
    yo, A = c.oracle()
    _assert_close(y, yo, A)
    for t in range(m):
        y1 = c.gpu(fg, Wd=flat, row_bytes=rb, qs=to_dev(c.qs[t:t + 1]), d=to_dev(c.d[t:t + 1]), m=1)
        assert y[t].tobytes() == y1[0].tobytes(), t
    vec, mat = (("k_gemv_q8_0_fast", "k_gemv_q8_0_mfma") if kind == "q8_0"
                else ("k_gemv_e4m3<", "k_gemv_e4m3_mfma<"))
    rbf = (lambda n: n // 32 * 34) if kind == "q8_0" else (lambda n: n)
    assert fg.gemv_launch_info(kind + "_mc", rb, m, in_f, out_f)["kernel"].startswith(vec)
    assert fg.gemv_launch_info(kind + "_mc", rbf(in_f), m, in_f, out_f)["kernel"].startswith(mat)
    assert fg.gemv_launch_info(kind + "_mc", rbf(65536), m, 65536, out_f)["kernel"].startswith(mat)
    assert fg.gemv_launch_info(kind, rbf(in_f), m, in_f, out_f)["kernel"].startswith(vec)


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_matrix_core_rows_independent_of_order(fg, kind):
    # the same 8 rows in reverse order give each row the same bits
    case(f"{kind} matrix cores, rows reversed")
    c = Case(kind, 300, 5120, 8)
    y = c.gpu(fg, mc=True)
    rev = list(range(7, -1, -1))
    yr = c.gpu(fg, qs=to_dev(c.qs[rev]), d=to_dev(c.d[rev]), mc=True)
    assert y.tobytes() == yr[rev].tobytes()


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_matrix_core_padded_row_stride(fg, kind):
    case(f"{kind} matrix cores, padded row stride")
    out_f, in_f, m = 100, (1024 if kind == "q8_0" else 1056), 5
    c = Case(kind, out_f, in_f, m)
    pad = 48
    Wp = np.zeros((out_f, c.row_bytes + pad), dtype=np.uint8)
    Wp[:, :c.row_bytes] = c.W
    Wp[:, c.row_bytes:] = 0x7F  # NaN codes, never read
    y = c.gpu(fg, Wd=to_dev(Wp), row_bytes=c.row_bytes + pad, mc=True)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_rotated_copies_are_identical(fg, kind):
    case(f"{kind} rotated copies")
    c = Case(kind, 5120, 5120, 1)
    ys = [c.gpu(fg, Wd=to_dev(c.W)).tobytes() for _ in range(3)]
    assert ys[0] == ys[1] == ys[2]


def test_e4m3_decode_on_device_exhaustive(fg):
    # Row r holds code r (0x7F / 0xFF excluded) in column 0 and zeros elsewhere; a one-hot
    # activation with d = 1 reads that column, so y[r] is the decoded code exactly.
    case("e4m3 decode through gemv_e4m3_q81 / blk128")
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    in_f = 32
    W = np.zeros((len(codes), in_f), dtype=np.uint8)
    W[:, 0] = codes
    qs = np.zeros((1, in_f), dtype=np.int8)
    qs[0, 0] = 1
    d = np.ones((1, 1), dtype=np.float32)
    y = torch.empty((1, len(codes)), device=dev())
    fg.gemv_e4m3_q81(to_dev(W), in_f, 1.0, to_dev(qs), to_dev(d), y, 1, in_f, len(codes))
    want = np.array([oracle.e4m3_value(c) for c in codes])
    assert np.array_equal(host(y)[0].astype(np.float64), want)
    grid = np.ones(((len(codes) + 127) // 128, 1), dtype=np.float32)
    fg.gemv_e4m3_blk128_q81(to_dev(W), in_f, to_dev(grid), 1, to_dev(qs), to_dev(d), y, 1, in_f,
                            len(codes))
    assert np.array_equal(host(y)[0].astype(np.float64), want)


@pytest.mark.parametrize("in_f", [2048, 288])
def test_q8_0_unaligned_rows_take_the_generic_path(fg, in_f):
    # W 2-byte aligned but not 16-byte aligned (and in_f % 256 != 0 for 288): generic path.
    case(f"q8_0 generic path in_f={in_f}")
    c = Case("q8_0", 77, in_f, 2)
    flat = np.zeros(c.W.size + 16, dtype=np.uint8)
    flat[2:2 + c.W.size] = c.W.reshape(-1)
    buf = to_dev(flat)
    y = c.gpu(fg, Wd=buf[2:])
    yo, A = c.oracle()
    _assert_close(y, yo, A)
    assert y.tobytes() == c.gpu(fg, Wd=buf[2:]).tobytes()


# Q8_0 row layouts the matrix-core kernel does not take (in_f % 256 != 0, or W only 2-byte
# aligned): the matrix-core entry point runs the plain entry point's kernels, so its rows are
# byte-identical to the plain call's, for m = 1 and for several rows.
@pytest.mark.parametrize("in_f,offset", [(288, 0), (1056, 0), (2048, 2)])
@pytest.mark.parametrize("m", [1, 5])
def test_q8_0_matrix_core_entry_falls_back_off_its_layouts(fg, in_f, offset, m):
    case(f"q8_0 matrix-core entry fallback in_f={in_f} offset={offset} m={m}")
    c = Case("q8_0", 77, in_f, m)
    flat = np.zeros(c.W.size + 16, dtype=np.uint8)
    flat[offset:offset + c.W.size] = c.W.reshape(-1)
    Wd = to_dev(flat)[offset:]
    y = c.gpu(fg, Wd=Wd, mc=True)
    assert y.tobytes() == c.gpu(fg, Wd=Wd).tobytes()
    yo, A = c.oracle()
    _assert_close(y, yo, A)
    kern = fg.gemv_launch_info("q8_0_mc", c.row_bytes, m, in_f, 77,
                               w_align=2 if offset else 256)["kernel"]
    assert "mfma" not in kern


@pytest.mark.parametrize("kind", ["e4m3", "blk128", "q8_0"])
def test_padded_row_stride(fg, kind):
    case(f"{kind} padded row stride")
    out_f, in_f = 100, 1024
    c = Case(kind, out_f, in_f, 1)
    pad = 48
    Wp = np.zeros((out_f, c.row_bytes + pad), dtype=np.uint8)
    Wp[:, :c.row_bytes] = c.W
    Wp[:, c.row_bytes:] = 0x7F  # never read
    y = c.gpu(fg, Wd=to_dev(Wp), row_bytes=c.row_bytes + pad)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


@pytest.mark.parametrize("kind", KINDS)
def test_max_in_f(fg, kind):
    case(f"{kind} in_f=65536")
    c = Case(kind, 40, 65536, 1)
    y = c.gpu(fg)
    yo, A = c.oracle()
    _assert_close(y, yo, A)


# The largest m the library accepts (the launch grid's y dimension indexes activation rows):
# in_f = 256 takes the Q8_0 fast path, and m = 65535 is 8192 passes of 8 rows, the last one
# with a single row.  Every output against the oracle, and sampled rows bit-identical to the
# same row computed alone.
@pytest.mark.parametrize("kind", KINDS)
def test_max_m(fg, kind):
    m, out_f, in_f = 65535, 5, 256
    case(f"{kind} m={m} out_f={out_f} in_f={in_f}")
    c = Case(kind, out_f, in_f, m)
    y = c.gpu(fg)
    yo, A = c.oracle()
    _assert_close(y, yo, A)
    for t in (0, 1, 7, 8, 32767, m - 2, m - 1):
        assert row_reference(fg, c, t).tobytes() == y[t].tobytes(), f"row {t}"
    # the matrix-core entry point over the same 65535 rows (8192 passes of 8)
    y = c.gpu(fg, mc=True)
    _assert_close(y, yo, A)
    for t in (0, 7, 8, m - 1):
        assert row_reference(fg, c, t, mc=True).tobytes() == y[t].tobytes(), f"row {t}"


def test_bad_arguments_raise_and_launch_nothing(fg):
    case("argument errors through the binding")
    c = Case("e4m3", 64, 256, 1)
    y = torch.zeros((1, 64), device=dev())
    with pytest.raises(fg.Fp8GemvError) as e:
        fg.gemv_e4m3_q81(c.Wd, 128, 1.0, to_dev(c.qs), to_dev(c.d), y, 1, 256, 64)
    assert e.value.rc == fg.FP8GEMV_ERR_ROW_BYTES
    with pytest.raises(fg.Fp8GemvError):
        fg.gemv_e4m3_blk128_q81(c.Wd, 256, to_dev(np.ones((1, 5), np.float32)), 5,
                                to_dev(c.qs), to_dev(c.d), y, 1, 256, 64)
    assert np.all(host(y) == 0)


def test_one_hip_runtime_in_process(fg):
    torch.zeros(1, device=dev())
    maps = open(f"/proc/{os.getpid()}/maps").read().splitlines()
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_graph_replays_match_eager(fg):
    # The bench replays the hot path from a HIP graph: every replay, with eager work and
    # synchronisations between replays, must reproduce the eager bytes.
    case("graph replay of producer + three GEMVs")
    in_f, out_f = 2048, 768
    x = to_dev(synth.x_rows(in_f, 1))
    w = to_dev(synth.gain(in_f))
    qs = torch.empty((1, in_f), dtype=torch.int8, device=dev())
    d = torch.empty((1, in_f // 32), device=dev())
    cases = [Case(k, out_f, in_f, 1) for k in KINDS]
    ys = [torch.empty((1, out_f), device=dev()) for _ in KINDS]

    def run():
        fg.rmsnorm_q8_1(x, w, None, qs, d, in_f, 1)
        for c, y in zip(cases, ys):
            if c.kind == "q8_0":
                fg.gemv_q8_0_q81(c.Wd, c.row_bytes, qs, d, y, 1, in_f, out_f)
            elif c.kind == "e4m3":
                fg.gemv_e4m3_q81(c.Wd, c.row_bytes, SCALE, qs, d, y, 1, in_f, out_f)
            else:
                fg.gemv_e4m3_blk128_q81(c.Wd, c.row_bytes, c.gd, c.grid.shape[1], qs, d, y, 1,
                                        in_f, out_f)

    run()
    eager = [host(y).copy() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        qs.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = [host(y) for y in ys]
        for e, gy in zip(eager, got):
            assert e.tobytes() == gy.tobytes(), rep
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replays_of_the_other_entry_points(fg):
    # The two-launch chains, the SiLU-gated and KDA gated-norm producers, m = 4 rows (plain and
    # matrix-core entry points) and the requantiser under graph replay: every replay, with eager work
    # between replays, reproduces the eager bytes.
    case("graph replay of chains, silu and gated producers, m = 4 and requant")
    in_f, out_f = 2048, 384
    x = to_dev(synth.x_rows(in_f, 4))
    w = to_dev(synth.gain(in_f))
    gate, up = to_dev(synth.f32(5, in_f)), to_dev(synth.f32(6, in_f))
    z = torch.empty((4, in_f), device=dev())
    qs = torch.empty((4, in_f), dtype=torch.int8, device=dev())
    d = torch.empty((4, in_f // 32), device=dev())
    h = torch.empty(in_f, device=dev())
    hq = torch.empty(in_f, dtype=torch.int8, device=dev())
    hd = torch.empty(in_f // 32, device=dev())
    go, gg, gw = to_dev(synth.f32(7, in_f)), to_dev(synth.f32(8, in_f)), to_dev(synth.gain(128))
    gz = torch.empty(in_f, device=dev())
    gq = torch.empty(in_f, dtype=torch.int8, device=dev())
    gdd = torch.empty(in_f // 32, device=dev())
    c = Case("blk128", out_f, in_f, 1)
    y = torch.empty((4, out_f), device=dev())
    Wq = torch.empty(out_f * in_f // 32 * 34, dtype=torch.uint8, device=dev())
    yq = torch.empty((4, out_f), device=dev())
    ymc = torch.empty((4, out_f), device=dev())
    yqmc = torch.empty((4, out_f), device=dev())
    outs = [z, qs, d, h, hq, hd, gz, gq, gdd, y, Wq, yq, ymc, yqmc]

    def run():
        fg.rms_norm_f32(x, w, z, in_f, 4)
        fg.quantize_q8_1(z, qs, d, 4, in_f)
        fg.silu_mul_q8_1(gate, up, h, hq, hd, in_f, 1)
        fg.gated_rmsnorm_q8_1(go, gg, gw, gz, gq, gdd, in_f, 128, 1)
        fg.gemv_e4m3_blk128_q81(c.Wd, c.row_bytes, c.gd, c.grid.shape[1], qs, d, y, 4, in_f,
                                out_f)
        fg.requant_e4m3_blk128_q8_0(c.Wd, c.row_bytes, c.gd, c.grid.shape[1], Wq,
                                    in_f // 32 * 34, in_f, out_f)
        fg.gemv_q8_0_q81(Wq, in_f // 32 * 34, qs, d, yq, 4, in_f, out_f)
        fg.gemv_e4m3_blk128_q81_mc(c.Wd, c.row_bytes, c.gd, c.grid.shape[1], qs, d, ymc, 4,
                                   in_f, out_f)
        fg.gemv_q8_0_q81_mc(Wq, in_f // 32 * 34, qs, d, yqmc, 4, in_f, out_f)

    run()
    eager = [host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        for e, t in zip(eager, outs):
            assert e.tobytes() == host(t).tobytes(), rep
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_read_bytes_measurement_kernel_runs(fg):
    case("fp8gemv_read_bytes")
    buf = torch.randint(0, 255, (3 * 32768 + 48,), dtype=torch.uint8, device=dev())
    sink = torch.full((1,), 7, dtype=torch.int32, device=dev())
    for nbytes in (16, 1000 * 16, buf.numel()):
        fg.fp8gemv_read_bytes(buf, nbytes, sink)
    assert int(host(sink)[0]) == 7


@pytest.mark.parametrize("pattern", ["chunk8k", "chunk16k", "wg8", "wg16", "persistent",
                                     "cached", "rows_1k", "rows_816", "empty", "one_wave",
                                     "rows_aligned", "line_windows"])
def test_read_patterns_run(fg, pattern):
    # Every measurement pattern over ragged and whole ranges; the rows patterns over rows of
    # 5120 and 5440 bytes (the e4m3 and Q8_0 rows at in_f = 5120).  Nothing is computed, so
    # the check is that each launch completes and leaves the sink alone.
    case(f"fp8gemv_read_pattern {pattern}")
    buf = torch.randint(0, 255, (64 * 5440,), dtype=torch.uint8, device=dev())
    sink = torch.full((1,), 7, dtype=torch.int32, device=dev())
    if pattern.startswith("rows") or pattern == "line_windows":
        for rb in (5120, 5440):
            for rows in (1, 5, 64):
                fg.fp8gemv_read_pattern(buf, rows * rb, pattern, sink, row_bytes=rb)
    else:
        for nbytes in (16, 1000 * 16, 33 * 1024 + 48, buf.numel()):
            fg.fp8gemv_read_pattern(buf, nbytes, pattern, sink)
    assert int(host(sink)[0]) == 7


def test_calls_on_an_explicit_stream_are_ordered_on_it(fg):
    # Every entry point takes the caller's stream: a producer -> GEMV chain issued on a
    # non-default stream runs there in order and matches the same chain on the default one.
    case("explicit stream")
    in_f, out_f = 4096, 1000
    x = to_dev(synth.x_rows(in_f, 1))
    w = to_dev(synth.gain(in_f))
    c = Case("q8_0", out_f, in_f, 1)
    outs = []
    for use_side in (False, True):
        s = torch.cuda.Stream() if use_side else torch.cuda.current_stream()
        qs = torch.empty(in_f, dtype=torch.int8, device=dev())
        d = torch.empty(in_f // 32, device=dev())
        y = torch.empty(out_f, device=dev())
        torch.cuda.synchronize()
        fg.rmsnorm_q8_1(x, w, None, qs, d, in_f, 1, stream=s)
        fg.gemv_q8_0_q81(c.Wd, c.row_bytes, qs, d, y, 1, in_f, out_f, stream=s)
        s.synchronize()
        outs.append(host(y).tobytes())
    assert outs[0] == outs[1]


def _q8_0_rows(out_f, in_f, rng, scale_bits=None, q=None):
    nb = in_f // 32
    W = np.zeros((out_f, nb * 34), dtype=np.uint8)
    for r in range(out_f):
        for b in range(nb):
            h = scale_bits(r, b) if scale_bits else 0x1400
            W[r, 34 * b] = h & 0xFF
            W[r, 34 * b + 1] = h >> 8
            W[r, 34 * b + 2:34 * b + 34] = (q(r, b) if q else
                                            rng.integers(-128, 128, 32)).astype(np.int8).view(np.uint8)
    return W


def test_gemv_degenerate_values(fg):
    # The degenerate cases of the containers and the activation, against the oracle:
    # Q8_0 quants of -128 and fp16 block scales at the largest normal, a subnormal and zero;
    # e4m3 weights of -0.0 and +-448; activation blocks with d = 0 and with qs = +-127;
    # a block-128 grid with zero and large tiles.
    case("gemv degenerate values")
    rng = np.random.default_rng(17)
    out_f, in_f = 70, 1024  # fast paths (in_f % 256 == 0), two 1 KiB windows
    x = synth.x_rows(in_f, 2)
    qs, d = oracle.quantize_q8_1(x)
    qs[0, 64:96] = 0
    d[0, 2] = 0.0                      # a block with d = 0
    qs[1, :32] = 127
    qs[1, 32:64] = -127                # saturated blocks
    d[1, 5] = 0.0
    qsd, dd = to_dev(qs), to_dev(d)
    scales = [0x7BFF, 0x0001, 0x0000, 0x3C00, 0x8400, 0x1400]  # 65504, 2^-24, 0, 1, -2^-14

    def sb(r, b):
        return scales[(r + b) % len(scales)]
    Wq = _q8_0_rows(out_f, in_f, rng, scale_bits=sb,
                    q=lambda r, b: np.full(32, -128) if (r + 2 * b) % 7 == 0 else
                    rng.integers(-128, 128, 32))
    y = torch.empty((2, out_f), device=dev())
    fg.gemv_q8_0_q81(to_dev(Wq), Wq.shape[1], qsd, dd, y, 2, in_f, out_f)
    yo, A = oracle.gemv_q8_0(Wq, Wq.shape[1], qs, d, in_f, out_f)
    _assert_close(host(y), yo, A)

    We = synth.e4m3_weights(out_f, in_f).copy()
    We[1::5, ::7] = 0x7E                # +448
    We[2::5, 3::7] = 0xFE               # -448
    We[::3, :] = 0x80                   # whole rows of -0.0
    fg.gemv_e4m3_q81(to_dev(We), in_f, 1.0, qsd, dd, y, 2, in_f, out_f)
    yo, A = oracle.gemv_e4m3(We, in_f, 1.0, qs, d, in_f, out_f)
    yh = host(y)
    _assert_close(yh, yo, A)
    assert np.all(yh[:, ::3] == 0.0)

    grid = synth.blk128_grid(out_f, in_f).copy()
    grid[0, 1] = 0.0
    grid[0, 3] = 2.0 ** 20
    fg.gemv_e4m3_blk128_q81(to_dev(We), in_f, to_dev(grid), grid.shape[1], qsd, dd, y, 2, in_f,
                            out_f)
    yo, A = oracle.gemv_e4m3_blk128(We, in_f, grid, qs, d, in_f, out_f)
    _assert_close(host(y), yo, A)
