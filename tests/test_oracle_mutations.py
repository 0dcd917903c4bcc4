"""Mutation check of the oracle: every planted slip must fail a pin.

Each case copies the oracle package (``oracle.c`` and ``__init__.py``) into a scratch folder,
plants one plausible mistake in the copy (a wrong exponent or bias in a decoder, swapped bytes,
a shifted index, a dropped scale or eps, another rounding rule, a sign), and runs the pin tests
of ``test_oracle_pins.py`` against that copy in a fresh process.  The case passes when at least
one pin fails.  The unmodified copy must pass every pin, so a failure comes from the slip and
not from the copying.  Everything here runs on the CPU; the HIP library is not involved.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, file in the oracle package, text, replacement, which occurrence of the text)
# Not listed: ties to even in the requantiser's q = round(v * id).  Its only exact ties are
# |v * id| = 63.5, at an element of exactly half the block maximum, where both rules give 64
# (test_requant_meets_ties_only_at_half_the_maximum), so that slip computes the same function.
MUTANTS = [
    # decoders
    ("e4m3 subnormal exponent", "oracle.c", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)", 0),
    ("e4m3 exponent bias", "oracle.c", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", 0),
    ("fp16 subnormal exponent", "oracle.c", "ldexp((double)m / 1024.0, -14)", "ldexp((double)m / 1024.0, -15)", 0),
    ("fp16 exponent bias", "oracle.c", "ldexp(1.0 + (double)m / 1024.0, e - 15)", "ldexp(1.0 + (double)m / 1024.0, e - 14)", 0),
    # q8_1 quantiser
    ("q8_1 ties to even", "oracle.c", "(int8_t)roundf(v);", "(int8_t)rintf(v);", 0),
    ("q8_1 amax / 128", "oracle.c", "amax / 127.0f", "amax / 128.0f", 0),
    ("q8_1 signed max", "oracle.c", "float a = fabsf(zb[i]);", "float a = zb[i];", 0),
    ("q8_1 quotient instead of reciprocal", "oracle.c", "float v = zb[i] * id;", "float v = zb[i] / db;", 0),
    # GEMVs
    ("Q8_0 scale bytes swapped", "oracle.c", "(blk[0] | (blk[1] << 8))", "(blk[1] | (blk[0] << 8))", 0),
    ("Q8_0 quant index shifted", "oracle.c", "blk[2 + k % 32]", "blk[1 + k % 32]", 0),
    ("Q8_0 activation index shifted", "oracle.c", "(double)qs[(int64_t)t * in_f + k]",
     "(double)qs[(int64_t)t * in_f + (k + 1) % in_f]", 0),
    ("e4m3 activation scale index shifted", "oracle.c", "d[(int64_t)t * nb + k / 32]",
     "d[(int64_t)t * nb + (k / 32 + 1) % nb]", 1),
    ("e4m3 per-tensor scale dropped", "oracle.c", "double w_hat = (double)scale * wv;", "double w_hat = wv;", 0),
    ("block-128 grid column shifted", "oracle.c", "grid[(int64_t)(r / 128) * grid_cols + k / 128]",
     "grid[(int64_t)(r / 128) * grid_cols + (k / 128 + 1) % grid_cols]", 0),
    ("block-128 grid ignored", "oracle.c", "double g = (double)grid[(int64_t)(r / 128) * grid_cols + k / 128];",
     "double g = 1.0;", 0),
    # requantiser and binary16 rounding
    ("requant quotient instead of reciprocal", "oracle.c", "(int8_t)roundf(v[i] * id)", "(int8_t)roundf(v[i] / db)", 0),
    ("requant amax / 128", "oracle.c", "amax / 127.0f", "amax / 128.0f", 1),
    ("requant against the fp16 scale", "oracle.c", "float id = (db != 0.0f) ? 1.0f / db : 0.0f;",
     "float id = (db != 0.0f) ? 1.0f / (float)oracle_fp16_value(oracle_f32_to_fp16(db)) : 0.0f;", 1),
    ("requant grid column shifted", "oracle.c", "grid_cols + (32 * b) / 128]", "grid_cols + ((32 * b) / 128 + 1) % grid_cols]", 0),
    ("requant scale bytes swapped", "oracle.c", "out[34 * b] = (uint8_t)(h & 0xFF);", "out[34 * b] = (uint8_t)(h >> 8);", 0),
    ("binary16 ties away from zero", "oracle.c", "return fmod(r, 2.0) == 0.0 ? r : r + 1.0;", "return r + 1.0;", 0),
    # SiLU-gated product
    ("silu sign of the exponent", "oracle.c", "g / (1.0 + exp(-g))", "g / (1.0 + exp(g))", 0),
    ("silu as a plain sigmoid", "oracle.c", "g / (1.0 + exp(-g))", "1.0 / (1.0 + exp(-g))", 0),
    ("silu up factor dropped", "oracle.c", "double h = sg * (double)up[i];", "double h = sg;", 0),
    ("silu rounded to f32 before the product", "oracle.c", "double h = sg * (double)up[i];",
     "double h = (double)(float)sg * (double)up[i];", 0),
    # RMSNorm and the KDA gated norm (Python, f64)
    ("rmsnorm eps dropped", "__init__.py", "math.sqrt(ss / ncols + eps64)", "math.sqrt(ss / ncols)", 0),
    ("rmsnorm divides by n - 1", "__init__.py", "math.sqrt(ss / ncols + eps64)", "math.sqrt(ss / (ncols - 1) + eps64)", 0),
    ("rmsnorm without the square root", "__init__.py", "1.0 / math.sqrt(ss / ncols + eps64)", "1.0 / (ss / ncols + eps64)", 0),
    ("gated norm gate sign", "__init__.py", "1.0 / (1.0 + _exp(-v))", "1.0 / (1.0 + _exp(v))", 0),
    ("gated norm divides by n - 1", "__init__.py", "math.sqrt(ss / head_dim + eps64)", "math.sqrt(ss / (head_dim - 1) + eps64)", 0),
    ("gated norm gate dropped", "__init__.py", "((o64[r, sl] * w64) * s) * gate", "((o64[r, sl] * w64) * s)", 0),
]

# Imports the oracle copy first, so the pin module's ``import oracle`` finds it in sys.modules.
RUNNER = (
    "import sys\n"
    "sys.path.insert(0, sys.argv[1])\n"
    "import oracle\n"
    "assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__\n"
    "import pytest\n"
    "sys.exit(pytest.main([sys.argv[2], '-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu']))\n"
)


def _replace_nth(text: str, old: str, new: str, nth: int) -> str:
    at = -1
    for _ in range(nth + 1):
        at = text.find(old, at + 1)
        assert at >= 0, f"{old!r}: occurrence {nth} not found"
    return text[:at] + new + text[at + len(old):]


def _run(case, scratch: str):
    """Returns (name, pins passed?, tail of the pytest output)."""
    name, fname, old, new, nth = case
    d = os.path.join(scratch, "m%02d" % (MUTANTS.index(case) + 1 if case in MUTANTS else 0))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp"))
    if fname:
        p = os.path.join(d, "oracle", fname)
        with open(p) as f:
            text = f.read()
        with open(p, "w") as f:
            f.write(_replace_nth(text, old, new, nth))
    r = subprocess.run([sys.executable, "-c", RUNNER, d, PINS], cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    return name, r.returncode == 0, (r.stdout + r.stderr)[-1500:]


def test_every_planted_slip_fails_a_pin():
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as scratch:
        control = ("unmodified copy", "", "", "", 0)
        with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as pool:
            futs = [pool.submit(_run, control, scratch)]
            futs += [pool.submit(_run, m, scratch) for m in MUTANTS]
            results = [f.result() for f in futs]
    name, passed, tail = results[0]
    assert passed, f"the unmodified oracle copy fails its pins:\n{tail}"
    survivors = [(n, t) for n, ok, t in results[1:] if ok]
    assert not survivors, "slips no pin catches: " + ", ".join(n for n, _ in survivors)


@pytest.mark.parametrize("case", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_each_slip_applies_once_where_meant(case):
    """Every planted slip names text that exists in the oracle, so no case is a no-op."""
    _, fname, old, new, nth = case
    with open(os.path.join(ROOT, "oracle", fname)) as f:
        text = f.read()
    assert text.count(old) > nth
    assert _replace_nth(text, old, new, nth) != text


def test_requant_meets_ties_only_at_half_the_maximum():
    """v * 127 / amax is a ratio of two e4m3 values times 127, and 127 is prime, so it is a
    half-integer only at v = amax / 2 (63.5); the f32 steps move it by a few parts in 2^24,
    far less than its distance to any other half-integer.  So every exact tie of the
    requantiser's f32 product is +-63.5, where halves away from zero and ties to even agree.
    Checked over every pair of e4m3 codes (block maximum, element) at dyadic and inexact
    scales, with the oracle's f32 steps."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    f32 = np.float32
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([oracle.e4m3_value(c) for c in codes], dtype=np.float32)
    scales = [1.0, 2.0 ** -20, 2.0 ** 6, 0.3, 0.7, 1.1, 3.0, 1e-30]
    ties = 0
    for S in np.array(scales, dtype=np.float32):
        v = (vals * S).astype(np.float32)
        for i in np.nonzero(vals > 0)[0]:
            d = f32(v[i] / f32(127))
            if d == 0:
                continue
            inv = f32(f32(1) / d)
            if not np.isfinite(inv):
                continue
            t = np.abs((v[np.abs(vals) <= vals[i]] * inv).astype(np.float32))
            at = t[t - np.floor(t) == 0.5]
            ties += at.size
            assert np.all(at == 63.5), (float(S), codes[i], sorted(set(at.tolist())))
    assert ties > 0  # the half-maximum ties are met, so the check is not vacuous
