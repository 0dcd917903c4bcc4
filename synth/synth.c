/*
 * Seeded synthetic inputs for the m=1 decode matvec: x / gain rows, raw e4m3 weight planes,
 * ggml Q8_0 weight rows and block-128 f32 scale grids.
 *
 * This file holds no arithmetic of the method itself (no normalisation, quantisation, decode
 * or dot product); it only draws bytes and floats.  Both the HIP library's tests/bench and the
 * CPU oracle consume what it writes, so it must stay free of either side's code.
 *
 * Generator: xorshift64 with shifts 13 / 7 / 17 and state = seed | 1, the generator the
 * fused-producer gate page (q8_fuse_gate.rs, `Xorshift64`) uses for its x and w rows.  Every
 * value is taken from the high bits of one 64-bit draw:
 *   f32 in [-4, 4)   : ((r >> 40) / 2^24 - 0.5) * 8, redrawn when it would be exactly 0
 *   e4m3 byte        : magnitude r >> 57 (7 bits; 0x7F, the NaN code, becomes 0x30), sign bit (r >> 56) & 1
 *   int8 [-127, 127] : ((r >> 32) % 255) - 127
 *   fp16 scale       : 2^-8 + u * (2^-4 - 2^-8), u = (r >> 40) / 2^24, rounded to nearest-even fp16
 *   grid value       : 2^(-6 + ((r >> 32) % 5))
 */
#include <stdint.h>
#include <math.h>
#include <string.h>

static inline uint64_t xs_next(uint64_t *s) {
    uint64_t x = *s;
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    *s = x;
    return x;
}

/* f32 uniform on the 2^-21 grid of [-4, 4), never exactly zero. */
static inline float xs_f32(uint64_t *s) {
    for (;;) {
        uint32_t bits = (uint32_t)(xs_next(s) >> 40);
        if (bits == (1u << 23)) continue; /* would give exactly 0.0 */
        float unit = (float)bits / 16777216.0f;
        return (unit - 0.5f) * 8.0f;
    }
}

void synth_f32(uint64_t seed, float *out, int64_t n) {
    uint64_t s = seed | 1u;
    for (int64_t i = 0; i < n; ++i) out[i] = xs_f32(&s);
}

/* Raw e4m3 bytes, uniform 7-bit magnitude with 0x7F replaced by 0x30, random sign. */
void synth_e4m3(uint64_t seed, uint8_t *out, int64_t n) {
    uint64_t s = seed | 1u;
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = xs_next(&s);
        uint8_t mag = (uint8_t)(r >> 57);
        if (mag == 0x7F) mag = 0x30;
        out[i] = (uint8_t)(mag | (((r >> 56) & 1u) << 7));
    }
}

/* Round a positive, normal-range double to the nearest-even binary16 bit pattern. */
static uint16_t to_fp16_bits(double v) {
    int e;
    double m = frexp(v, &e);          /* v = m * 2^e, m in [0.5, 1) */
    double sig = m * 2048.0;           /* [1024, 2048): 11 significant bits */
    double r = nearbyint(sig);         /* default rounding mode: nearest-even */
    if (r >= 2048.0) { r = 1024.0; e += 1; }
    int exp16 = (e - 1) + 15;          /* v = (r / 1024) * 2^(e-1) */
    return (uint16_t)((exp16 << 10) | ((int)r - 1024));
}

/* ggml Q8_0 rows: per 32-weight block a little-endian fp16 scale then 32 int8. Blocks are
 * written back to back (row_bytes = in_f / 32 * 34). Per block: one draw for the scale, then
 * one draw per int8. */
void synth_q8_0(uint64_t seed, uint8_t *out, int64_t out_f, int64_t in_f) {
    uint64_t s = seed | 1u;
    int64_t nblk = out_f * (in_f / 32);
    for (int64_t b = 0; b < nblk; ++b) {
        uint8_t *blk = out + b * 34;
        double u = (double)(xs_next(&s) >> 40) / 16777216.0;
        double sc = 0.00390625 + u * (0.0625 - 0.00390625);
        uint16_t h = to_fp16_bits(sc);
        blk[0] = (uint8_t)(h & 0xFF);
        blk[1] = (uint8_t)(h >> 8);
        for (int i = 0; i < 32; ++i) {
            int v = (int)((xs_next(&s) >> 32) % 255u) - 127;
            blk[2 + i] = (uint8_t)(int8_t)v;
        }
    }
}

/* int8 values uniform in [-127, 127]. */
void synth_i8(uint64_t seed, int8_t *out, int64_t n) {
    uint64_t s = seed | 1u;
    for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)((int)((xs_next(&s) >> 32) % 255u) - 127);
}

/* Block-128 scale grid: powers of two 2^-6 .. 2^-2, log-uniform. */
void synth_grid(uint64_t seed, float *out, int64_t n) {
    uint64_t s = seed | 1u;
    for (int64_t i = 0; i < n; ++i) out[i] = ldexpf(1.0f, -6 + (int)((xs_next(&s) >> 32) % 5u));
}

/* Raw draws, for checking the generator itself against its published recurrence. */
void synth_raw_u64(uint64_t seed, uint64_t *out, int64_t n) {
    uint64_t s = seed | 1u;
    for (int64_t i = 0; i < n; ++i) out[i] = xs_next(&s);
}
