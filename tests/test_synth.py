"""The seeded generators: recurrence, ranges and determinism (host only)."""
import numpy as np

import synth


def _xorshift_ref(seed, n):
    s = (seed | 1) & (2 ** 64 - 1)
    out = []
    for _ in range(n):
        s ^= (s << 13) & (2 ** 64 - 1)
        s ^= s >> 7
        s ^= (s << 17) & (2 ** 64 - 1)
        out.append(s)
    return out


def test_xorshift64_recurrence():
    # q8_fuse_gate.rs, `Xorshift64`: shifts 13, 7, 17 on a state seeded with seed | 1.
    for seed in (0, 1, synth.SEED_X ^ 4096, 2 ** 64 - 1):
        assert synth.raw_u64(seed, 50).tolist() == _xorshift_ref(seed, 50)


def test_f32_draws_match_recipe_and_avoid_zero():
    seed = synth.SEED_X ^ 8192
    raw = _xorshift_ref(seed, 20000)
    want = [((r >> 40) / 2 ** 24 - 0.5) * 8 for r in raw if (r >> 40) != 2 ** 23]
    got = synth.f32(seed, len(want))
    assert got.astype(np.float64).tolist() == want
    x = synth.x_rows(8192, 3)
    assert x.min() >= -4 and x.max() < 4 and np.all(x != 0)
    assert np.array_equal(x[0], synth.x_rows(8192, 1)[0])   # row 0 is the m=1 input
    assert not np.array_equal(x[0], x[1])


def test_e4m3_bytes_have_no_nan_code():
    w = synth.e4m3_weights(64, 4096)
    assert not np.any((w & 0x7F) == 0x7F)
    counts = np.bincount(w.reshape(-1), minlength=256)
    assert counts[0x30] > counts[0x31]            # 0x30 also takes the NaN draws
    assert abs(counts[:128].sum() - counts[128:].sum()) < 0.01 * w.size


def test_q8_0_rows_ranges():
    out_f, in_f = 33, 2048
    W = synth.q8_0_weights(out_f, in_f)
    assert W.shape == (out_f, in_f // 32 * 34)
    blk = W.reshape(out_f, in_f // 32, 34)
    sc = blk[:, :, :2].copy().view(np.float16).astype(np.float64)
    assert sc.min() >= 2.0 ** -8 and sc.max() <= 2.0 ** -4
    q = blk[:, :, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127


def test_grid_values_are_the_five_powers_of_two():
    g = synth.blk128_grid(17408, 5120)
    assert g.shape == (136, 40)
    assert set(np.unique(g).tolist()) == {2.0 ** e for e in range(-6, -1)}


def test_generators_are_deterministic():
    assert np.array_equal(synth.e4m3_weights(8, 256), synth.e4m3_weights(8, 256))
    assert not np.array_equal(synth.e4m3_weights(8, 256), synth.e4m3_weights(8, 288)[:, :256])
