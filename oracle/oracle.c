/*
 * CPU oracle for the m=1 decode matvec path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's cpu_baseline leg may load this library.
 * It shares no code, header, table or helper with the HIP library and must never be used as
 * a fallback for it.  Everything here is the plain definition, written for a reader to check
 * by eye: no blocking, no fusion, no reordering, f64 accumulation.
 *
 * Sources (docs.rs pages of memra-engine 0.125.0):
 *   [gate]  src/bin/q8_fuse_gate.rs   -- module doc and `run_shape`: rms_norm -> quantize_q8_1
 *           chain, q8_1 = int8 qs plus an f32 scale per 32 values, the `id = 1/d` branch.
 *   [bench] src/bin/gemv_e4m3_bench.rs -- module doc (QUESTION, THE COMPARISON, THE BLOCK-128
 *           ARM) and `synth_e4m3`, `synth_blk_grid`, `synth_q8_0`: the three weight containers.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no FMA contraction, IEEE f32/f64).
 */
#include <math.h>
#include <stdint.h>

/* ---------------------------------------------------------------- decoders ---- */

/* OCP FP8 E4M3 (the "fn" variant: no infinities, NaN only at S.1111.111).  [bench]
 * `synth_e4m3`: magnitude 0x7F is the e4m3 NaN code and is excluded from weights.
 * Fields: sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
 *   exponent 0 : (-1)^s * (m / 8) * 2^-6        (subnormal)
 *   otherwise  : (-1)^s * (1 + m / 8) * 2^(e - 7)
 * Returns NaN for 0x7F / 0xFF. */
double oracle_e4m3_value(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* IEEE binary16 from its bit pattern (the fp16 scale at bytes 0..1 of a ggml block_q8_0,
 * little-endian).  [bench] `synth_q8_0`: 0x1400 is 2^-10.
 * Fields: sign = bit 15, exponent = bits 14..10 (bias 15), mantissa = bits 9..0. */
double oracle_fp16_value(uint16_t bits) {
    int s = bits >> 15;
    int e = (bits >> 10) & 31;
    int m = bits & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m / 1024.0, -14);
    else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -mag : mag;
}

/* --------------------------------------------------------------- quantiser ---- */

/* q8_1 quantisation of f32 rows z[nrows, ncols] (ncols a multiple of 32).  [gate] module doc
 * (int8 qs plus one f32 scale per 32 values) and the generator's note on the `id = 1/d`
 * branch.  Per 32-block, every operation in f32 (this decides an integer, so it is taken in
 * the kernel's precision):
 *   amax = max |z_i|
 *   d    = amax / 127
 *   id   = 1 / d   (0 when d == 0)
 *   q_i  = round(z_i * id), halves away from zero (C roundf)
 * Returns 0, -1 for a refused input (a block whose amax is nonzero but so small, below
 * 127 * 2^-128, that 1 / d overflows f32: the rule gives no integer there), or -2 when ncols
 * is not a multiple of 32. */
int oracle_quantize_q8_1(const float *z, int nrows, int ncols, int8_t *qs, float *d) {
    if (ncols % 32 != 0 || nrows < 0 || ncols < 0) return -2;
    int nb = ncols / 32;
    for (int r = 0; r < nrows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float *zb = z + (int64_t)r * ncols + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(zb[i]);
                if (a > amax) amax = a;
            }
            float db = amax / 127.0f;
            float id = (db != 0.0f) ? 1.0f / db : 0.0f;
            if (!isfinite(id)) return -1;
            for (int i = 0; i < 32; ++i) {
                float v = zb[i] * id;
                qs[(int64_t)r * ncols + 32 * b + i] = (int8_t)roundf(v);
            }
            d[(int64_t)r * nb + b] = db;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ GEMVs ---- */
/*
 * All three compute, for activation row t and weight row r,
 *     y[t, r] = sum_k  w_hat[r, k] * a_hat[t, k]          (k = 0 .. in_f-1, in order)
 *     A[t, r] = sum_k |w_hat[r, k] * a_hat[t, k]|
 * with the q8_1 activation a_hat[t, k] = d[t, k/32] * qs[t, k] and the container's
 * dequantised weight w_hat.  Terms and sums are f64.  Only weight rows r0 <= r < r1 are
 * computed (the caller samples rows); y and A are [m, out_f] row-major.
 * Return 0, -1 if a weight value is NaN/inf (refused input), -2 on bad shapes.
 */

static int check_shape(int m, int in_f, int out_f, int r0, int r1) {
    if (m < 1 || in_f < 32 || in_f % 32 != 0 || out_f < 1) return -2;
    if (r0 < 0 || r1 > out_f || r0 > r1) return -2;
    return 0;
}

/* [bench] THE COMPARISON, arm Q8_0: ggml block_q8_0 rows, 34 bytes per 32 weights -- an fp16
 * scale (little-endian, bytes 0..1) then 32 int8.  w_hat[r, k] = fp16(dw[r, k/32]) * qw[r, k]. */
int oracle_gemv_q8_0(const uint8_t *W, int64_t row_bytes, const int8_t *qs, const float *d,
                     int m, int in_f, int out_f, int r0, int r1, double *y, double *A) {
    int rc = check_shape(m, in_f, out_f, r0, r1);
    if (rc) return rc;
    int nb = in_f / 32;
    if (row_bytes < (int64_t)nb * 34) return -2;
    for (int t = 0; t < m; ++t) {
        for (int r = r0; r < r1; ++r) {
            const uint8_t *row = W + (int64_t)r * row_bytes;
            double acc = 0.0, aabs = 0.0;
            for (int k = 0; k < in_f; ++k) {
                const uint8_t *blk = row + (int64_t)(k / 32) * 34;
                double scale = oracle_fp16_value((uint16_t)(blk[0] | (blk[1] << 8)));
                if (!isfinite(scale)) return -1;
                double w_hat = scale * (double)(int8_t)blk[2 + k % 32];
                double a_hat = (double)d[(int64_t)t * nb + k / 32] * (double)qs[(int64_t)t * in_f + k];
                double term = w_hat * a_hat;
                acc += term;
                aabs += fabs(term);
            }
            y[(int64_t)t * out_f + r] = acc;
            A[(int64_t)t * out_f + r] = aabs;
        }
    }
    return 0;
}

/* [bench] THE COMPARISON, arm E4M3: raw e4m3 bytes [out_f, in_f], row stride row_bytes (in_f
 * on the page), one f32 per-tensor scale.  w_hat[r, k] = scale * e4m3(W[r, k]). */
int oracle_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                     const float *d, int m, int in_f, int out_f, int r0, int r1, double *y,
                     double *A) {
    int rc = check_shape(m, in_f, out_f, r0, r1);
    if (rc) return rc;
    int nb = in_f / 32;
    if (row_bytes < in_f) return -2;
    for (int t = 0; t < m; ++t) {
        for (int r = r0; r < r1; ++r) {
            const uint8_t *row = W + (int64_t)r * row_bytes;
            double acc = 0.0, aabs = 0.0;
            for (int k = 0; k < in_f; ++k) {
                double wv = oracle_e4m3_value(row[k]);
                if (isnan(wv)) return -1;
                double w_hat = (double)scale * wv;
                double a_hat = (double)d[(int64_t)t * nb + k / 32] * (double)qs[(int64_t)t * in_f + k];
                double term = w_hat * a_hat;
                acc += term;
                aabs += fabs(term);
            }
            y[(int64_t)t * out_f + r] = acc;
            A[(int64_t)t * out_f + r] = aabs;
        }
    }
    return 0;
}

/* [bench] THE BLOCK-128 ARM and `synth_blk_grid`: the same raw e4m3 plane plus an f32 grid
 * [ceil(out_f/128), ceil(in_f/128)], row-major with grid_cols = ceil(in_f/128) columns; the
 * grid value multiplies (a dequantisation factor).
 * w_hat[r, k] = grid[r/128, k/128] * e4m3(W[r, k]). */
int oracle_gemv_e4m3_blk128(const uint8_t *W, int64_t row_bytes, const float *grid,
                            int grid_cols, const int8_t *qs, const float *d, int m, int in_f,
                            int out_f, int r0, int r1, double *y, double *A) {
    int rc = check_shape(m, in_f, out_f, r0, r1);
    if (rc) return rc;
    int nb = in_f / 32;
    if (row_bytes < in_f || grid_cols != (in_f + 127) / 128) return -2;
    for (int t = 0; t < m; ++t) {
        for (int r = r0; r < r1; ++r) {
            const uint8_t *row = W + (int64_t)r * row_bytes;
            double acc = 0.0, aabs = 0.0;
            for (int k = 0; k < in_f; ++k) {
                double wv = oracle_e4m3_value(row[k]);
                double g = (double)grid[(int64_t)(r / 128) * grid_cols + k / 128];
                if (isnan(wv) || !isfinite(g)) return -1;
                double w_hat = g * wv;
                double a_hat = (double)d[(int64_t)t * nb + k / 32] * (double)qs[(int64_t)t * in_f + k];
                double term = w_hat * a_hat;
                acc += term;
                aabs += fabs(term);
            }
            y[(int64_t)t * out_f + r] = acc;
            A[(int64_t)t * out_f + r] = aabs;
        }
    }
    return 0;
}

/* ------------------------------------------------------------ requantiser ---- */

/* IEEE binary16 bit pattern of a finite f32, rounded to nearest with ties to even; results
 * below 2^-14 are subnormal, magnitudes from 65520 up round to infinity; NaN stays NaN.
 * Written from the binary16 definition: |f| = n * 2^(e-10) with 1024 <= n < 2048 (normal) or
 * n * 2^-24 with n < 1024 (subnormal); n is rounded, and a carry to 2048 moves to the next
 * exponent. */
static double round_half_even(double x) { /* x >= 0, exact in double */
    double r = floor(x), diff = x - r;
    if (diff > 0.5) return r + 1.0;
    if (diff < 0.5) return r;
    return fmod(r, 2.0) == 0.0 ? r : r + 1.0;
}

uint16_t oracle_f32_to_fp16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        double n = round_half_even(ldexp(a, 24)); /* 0 .. 1024; 1024 is the least normal */
        return sign | (uint16_t)n;
    }
    int ex;
    frexp(a, &ex); /* a = fr * 2^ex, 0.5 <= fr < 1, so 2^(ex-1) <= a < 2^ex */
    int e = ex - 1;
    double n = round_half_even(ldexp(a, 10 - e)); /* 1024 .. 2048 */
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0);
}

/*
 * Load-time requantisation of an e4m3 weight plane into ggml Q8_0 rows (the bench page's ship
 * path, QUESTION: FP8 checkpoints are dequantised to a Q8_0 slab at load, 34 bytes per 32
 * weights).  The page gives no formula.  The reading taken here is the one block rule the pages
 * do show for 32-value int8 blocks, the q8_1 quantiser of the gate page with its `id = 1/d`
 * branch, with the scale stored as fp16 (the Q8_0 container's scale type):
 *   v_i  = e4m3(W[r, 32b+i]) * S          f32 multiply; S = scale, or grid[r/128, b/4] when a
 *                                         block-128 grid is given (THE BLOCK-128 ARM)
 *   amax = max |v_i|,  d = amax / 127     f32
 *   id   = 1 / d  (0 when d == 0)         f32
 *   q_i  = round(v_i * id), halves away from zero
 *   block bytes: fp16(d) little-endian, then the 32 int8 q_i.
 * Rows r0 <= r < r1 are written at Wq + r * q_row_bytes.
 * Returns 0, -1 for a refused input (an e4m3 NaN code, a non-finite scale, or a block whose
 * d is so small that 1 / d overflows f32, which needs |S| below 2^-112), -2 on bad shapes.
 */
int oracle_requant_q8_0(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                        int grid_cols, uint8_t *Wq, int64_t q_row_bytes, int in_f, int out_f,
                        int r0, int r1) {
    if (in_f <= 0 || in_f % 32 != 0 || out_f < 1 || r0 < 0 || r1 > out_f || r0 > r1) return -2;
    int nb = in_f / 32;
    if (row_bytes < in_f || q_row_bytes < (int64_t)nb * 34) return -2;
    if (grid && grid_cols != (in_f + 127) / 128) return -2;
    for (int r = r0; r < r1; ++r) {
        const uint8_t *row = W + (int64_t)r * row_bytes;
        uint8_t *out = Wq + (int64_t)r * q_row_bytes;
        for (int b = 0; b < nb; ++b) {
            float S = grid ? grid[(int64_t)(r / 128) * grid_cols + (32 * b) / 128] : scale;
            if (!isfinite(S)) return -1;
            float v[32], amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                double e = oracle_e4m3_value(row[32 * b + i]);
                if (isnan(e)) return -1;
                v[i] = (float)e * S;
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            float db = amax / 127.0f;
            float id = (db != 0.0f) ? 1.0f / db : 0.0f;
            if (!isfinite(id)) return -1;
            uint16_t h = oracle_f32_to_fp16(db);
            out[34 * b] = (uint8_t)(h & 0xFF);
            out[34 * b + 1] = (uint8_t)(h >> 8);
            for (int i = 0; i < 32; ++i) {
                int8_t q = (int8_t)roundf(v[i] * id);
                out[34 * b + 2 + i] = (uint8_t)q;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------- SiLU-gated producer ---- */

/* h = silu(gate) * up for n values (q8_fuse_gate.rs `main`: the MoE expert-ff site's
 * silu/gate*up -> q8_1 producer; the page names the operation, not a formula).  The standard
 * SiLU-gated product, every step in f64 with libm exp, one rounding to f32:
 *   h64 = (g / (1 + exp(-g))) * u,   h32 = (float)h64.
 * The q8_1 step that follows is oracle_quantize_q8_1 on h32. */
void oracle_silu_mul(const float *gate, const float *up, int n, double *h64, float *h32) {
    for (int i = 0; i < n; ++i) {
        double g = (double)gate[i];
        double sg = g / (1.0 + exp(-g));
        double h = sg * (double)up[i];
        h64[i] = h;
        h32[i] = (float)h;
    }
}
