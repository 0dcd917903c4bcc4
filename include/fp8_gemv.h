/*
 * fp8_gemv.h -- C ABI of the MI355X (gfx950) m=1 decode matvec library.
 *
 * The library implements the hot path of single-token decode described on the docs.rs source
 * pages of memra-engine 0.125.0:
 *   - a producer that RMS-normalises an activation row and quantises it to q8_1
 *     (src/bin/q8_fuse_gate.rs: module doc, `run_shape`), and
 *   - GEMVs that stream a weight matrix once from HBM against that q8_1 activation, for three
 *     weight containers (src/bin/gemv_e4m3_bench.rs: module doc sections QUESTION,
 *     THE COMPARISON and THE BLOCK-128 ARM; `synth_e4m3`, `synth_blk_grid`, `synth_q8_0`).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer on the current HIP device, owned by the caller; the
 *     library never frees, retains or allocates memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the null
 *     stream) and never synchronises.  Buffers must stay alive until the stream reaches the
 *     launched work.
 *   - Return value: 0 on success; a negative FP8GEMV_ERR_* code when the arguments are
 *     invalid (checked on the host before anything is launched, so no GPU work is queued);
 *     a positive value is the hipError_t reported by the launch.
 *   - Sizes are elements unless named *_bytes.  Matrices are row-major.
 *   - q8_1 activation = two planes: qs int8 [rows, cols] and d f32 [rows, cols/32] (one
 *     scale per 32 consecutive values, d = amax/127; value = d * qs).  No per-block sum.
 *     A block whose amax is nonzero but below 127 * 2^-128 (about 3.7e-37) has no finite
 *     1 / d in f32; its qs are unspecified (documented, not checked).
 *   - Preconditions that are documented but not checked: no NaN/Inf in x, w, scales or grid;
 *     no e4m3 NaN code (0x7F, 0xFF) in a weight plane (the bench page's generator excludes
 *     it and says the real dispatch refuses it); buffers large enough for the sizes passed.
 */
#ifndef FP8_GEMV_H
#define FP8_GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes (negative: argument errors found on the host, nothing launched). */
#define FP8GEMV_OK              0
#define FP8GEMV_ERR_NULL       (-1) /* a required pointer is NULL */
#define FP8GEMV_ERR_SHAPE      (-2) /* cols/in_f not a positive multiple of 32, rows/m/out_f < 1 */
#define FP8GEMV_ERR_ROW_BYTES  (-3) /* row_bytes below the container minimum */
#define FP8GEMV_ERR_GRID       (-4) /* grid_cols != ceil(in_f / 128) */
#define FP8GEMV_ERR_ALIGN      (-5) /* a pointer or row stride breaks the stated alignment */
#define FP8GEMV_ERR_TOO_LARGE  (-6) /* a size beyond the stated limit */

/* Limits.  in_f (and the producer's ncols) is bounded so that one activation row staged in
 * LDS fits a workgroup; m (and the producer's nrows) is bounded by the launch grid's y
 * dimension, which indexes rows. */
#define FP8GEMV_MAX_IN_F   65536
#define FP8GEMV_MAX_M      65535

/*
 * rms_norm_f32 -- first half of the two-launch producer chain.
 * Source: q8_fuse_gate.rs, module doc and `run_shape` (rms_norm(x, w, z, ncols, nrows, eps)).
 * For each row r: z[r, j] = x[r, j] * w[j] / sqrt(mean_j(x[r, j]^2) + eps).
 *   x    f32 [nrows, ncols]   input rows
 *   w    f32 [ncols]          gain, broadcast over rows
 *   z    f32 [nrows, ncols]   output (may not alias x or w)
 *   ncols multiple of 32, <= FP8GEMV_MAX_IN_F; 1 <= nrows <= FP8GEMV_MAX_M; eps as given
 *   (1e-6 on the page)
 * Arithmetic: the sum of squares is accumulated in double-double and rounded once to f64,
 * s = 1 / sqrt(ss / ncols + eps) in f64, z = (float)((double)x * w * s).
 * Alignment: x, w, z 16-byte aligned.
 */
int rms_norm_f32(const float *x, const float *w, float *z, int ncols, int nrows, float eps,
                 void *stream);

/*
 * quantize_q8_1 -- second half of the chain; also the x -> q8_1 step in front of each GEMV.
 * Source: q8_fuse_gate.rs, module doc (int8 qs plus one f32 scale per 32 values) and the note
 * on the `id = 1/d` branch; gemv_e4m3_bench.rs, THE COMPARISON (the f32 activation is
 * quantised to q8_1 before the matvec).
 * Per 32-block, all in f32: amax = max|z|, d = amax / 127, id = (d != 0) ? 1 / d : 0,
 * qs = round(z * id) with halves away from zero.
 *   z   f32 [nrows, ncols]      input
 *   qs  int8 [nrows, ncols]     output
 *   d   f32 [nrows, ncols / 32] output
 * Argument order follows the page (nrows before ncols).  Limits as for rms_norm_f32.
 * Alignment: z and qs 16-byte aligned, d 4-byte aligned.
 */
int quantize_q8_1(const float *z, int8_t *qs, float *d, int nrows, int ncols, void *stream);

/*
 * rmsnorm_q8_1 -- the fused producer: rms_norm_f32 then quantize_q8_1 in one launch.
 * Source: q8_fuse_gate.rs, module doc (`rms_norm_zq8_f32`: one launch, still writes z, and
 * must be byte-identical in z, qs and d to the two-launch chain).
 * Same arguments and results as the chain; z may be NULL, in which case z is not stored
 * (qs and d are unchanged).  The bytes written are identical to rms_norm_f32 followed by
 * quantize_q8_1 on the same inputs.
 */
int rmsnorm_q8_1(const float *x, const float *w, float *z, int8_t *qs, float *d, int ncols,
                 int nrows, float eps, void *stream);

/*
 * silu_mul_f32 -- first half of the SiLU-gated producer chain: h = silu(gate) * up.
 * Source: q8_fuse_gate.rs, `main` (the MoE expert-ff width n_ff_exp = 1536 is the activation
 * fusion site, silu/gate*up -> q8_1, still on the unfused chain).  The page names the
 * operation and gives no formula; the rule is the standard SiLU-gated product:
 *   h[r, j] = (float)((g / (1 + exp(-g))) * u)  with g = gate[r, j], u = up[r, j] widened to
 *   f64, every step in f64, one rounding to f32 at the end.
 *   gate, up, h   f32 [nrows, ncols], 16-byte aligned; h may not alias gate or up
 *   ncols multiple of 32, <= FP8GEMV_MAX_IN_F; 1 <= nrows <= FP8GEMV_MAX_M
 * The chain is silu_mul_f32 then quantize_q8_1.
 */
int silu_mul_f32(const float *gate, const float *up, float *h, int ncols, int nrows,
                 void *stream);

/*
 * silu_mul_q8_1 -- the fused SiLU-gated producer: silu_mul_f32 then quantize_q8_1 in one
 * launch, byte-identical in h, qs and d to that chain.  h may be NULL (not stored).
 * Source: as above, with the fused-producer contract of q8_fuse_gate.rs's module doc.
 *   qs int8 [nrows, ncols] (16-byte aligned), d f32 [nrows, ncols / 32] (4-byte aligned)
 */
int silu_mul_q8_1(const float *gate, const float *up, float *h, int8_t *qs, float *d, int ncols,
                  int nrows, void *stream);

/*
 * gated_rms_norm_f32 -- first half of the KDA gated-norm producer chain.
 * Source: q8_fuse_gate.rs, module doc and `main` (the KDA qkv width, 64 heads x 128 head_dim
 * = 8192, is the KDA gated-norm site, still on the unfused chain).  The page gives no formula;
 * the rule is the output stage of a Kimi-delta-attention layer: RMSNorm over each head's
 * head_dim values, a gain shared by the heads, then the sigmoid output gate.  For each row r
 * and head h (columns h*head_dim .. h*head_dim + head_dim - 1), every step in f64 and one
 * rounding to f32 at the end:
 *   s = 1 / sqrt(sum_{j in h} o[r, j]^2 / head_dim + eps)
 *   z[r, j] = (float)(((o[r, j] * w[j mod head_dim]) * s) * (1 / (1 + exp(-g[r, j]))))
 *   o, g, z   f32 [nrows, ncols], 16-byte aligned; z may not alias o or g
 *   w         f32 [head_dim], 16-byte aligned
 *   head_dim  32, 64, 128 or 256;  ncols a multiple of 32 and of head_dim, <= FP8GEMV_MAX_IN_F;
 *             1 <= nrows <= FP8GEMV_MAX_M;  eps as for rms_norm_f32 (1e-6 on the page)
 * The chain is gated_rms_norm_f32 then quantize_q8_1.
 */
int gated_rms_norm_f32(const float *o, const float *g, const float *w, float *z, int ncols,
                       int head_dim, int nrows, float eps, void *stream);

/*
 * gated_rmsnorm_q8_1 -- the fused KDA gated-norm producer: gated_rms_norm_f32 then
 * quantize_q8_1 in one launch, byte-identical in z, qs and d to that chain.  z may be NULL
 * (not stored).  Source: as above, with the fused-producer contract of q8_fuse_gate.rs's
 * module doc.
 *   qs int8 [nrows, ncols] (16-byte aligned), d f32 [nrows, ncols / 32] (4-byte aligned)
 */
int gated_rmsnorm_q8_1(const float *o, const float *g, const float *w, float *z, int8_t *qs,
                       float *d, int ncols, int head_dim, int nrows, float eps, void *stream);

/*
 * gemv_q8_0_q81 -- matvec over ggml Q8_0 weight rows.
 * Source: gemv_e4m3_bench.rs, QUESTION and THE COMPARISON (arm Q8_0: 34 bytes per 32
 * weights, an fp16 scale then 32 int8, row_bytes = in_f / 32 * 34) and `synth_q8_0`.
 * y[t, r] = sum_b fp16(W[r].blk[b].d) * d_a[t, b] * sum_{i<32} W[r].blk[b].qs[i] * qs[t, 32b+i]
 *   W          [out_f] rows of row_bytes bytes; each row starts with in_f/32 blocks of 34 B
 *              (little-endian fp16 scale at bytes 0..1, then 32 int8)
 *   row_bytes  >= in_f / 32 * 34, even
 *   qs, d      q8_1 activation rows [m, in_f] / [m, in_f / 32]
 *   y          f32 [m, out_f]
 * Alignment: W and row_bytes 2-byte aligned; the fast path also needs W 16-byte aligned,
 * row_bytes % 16 == 0 and in_f % 256 == 0, otherwise a slower path runs.  qs, d 16-byte
 * aligned.  Each activation row is computed independently.  Every block's integer sum is
 * exact.  Up to 8 activation rows share one pass over the weights, and row t of an m-row
 * call is bit-identical to an m=1 call on that row, for every m (the batched arms' bit-parity
 * gate, gemv_e4m3_bench.rs, WHAT MADE THIS A BOUNDED WRITE).
 */
int gemv_q8_0_q81(const void *W, int64_t row_bytes, const int8_t *qs, const float *d, float *y,
                  int m, int in_f, int out_f, void *stream);

/*
 * gemv_e4m3_q81 -- matvec over raw OCP FP8 E4M3 weights with one per-tensor f32 scale.
 * Source: gemv_e4m3_bench.rs, THE COMPARISON (arm E4M3: the raw checkpoint bytes are the
 * weight stream, row_bytes == in_f, no dequantisation) and `synth_e4m3`.
 * y[t, r] = scale * sum_k e4m3(W[r, k]) * d_a[t, k/32] * qs[t, k]
 *   W          u8 [out_f] rows of row_bytes bytes (first in_f bytes used)
 *   row_bytes  >= in_f, multiple of 16;  W 16-byte aligned
 *   scale      per-tensor dequantisation factor, applied once per output
 *   qs, d, y   as for gemv_q8_0_q81
 * Each activation row is computed independently; up to 8 share one pass over the weights,
 * and row t of an m-row call is bit-identical to an m=1 call on that row, for every m.
 */
int gemv_e4m3_q81(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                  const float *d, float *y, int m, int in_f, int out_f, void *stream);

/*
 * gemv_e4m3_blk128_q81 -- matvec over raw e4m3 weights with a block-128 f32 scale grid.
 * Source: gemv_e4m3_bench.rs, THE BLOCK-128 ARM (an f32 [ceil(out_f/128), ceil(in_f/128)]
 * grid, the weight_scale_inv of weight_block_size [128, 128] checkpoints) and
 * `synth_blk_grid`.
 * y[t, r] = sum_k grid[r/128, k/128] * e4m3(W[r, k]) * d_a[t, k/32] * qs[t, k]
 *   grid       f32 [ceil(out_f/128), grid_cols], row-major, a multiplier
 *   grid_cols  must equal ceil(in_f / 128)
 *   other arguments, and the summation order for several activation rows, as for
 *   gemv_e4m3_q81
 */
int gemv_e4m3_blk128_q81(const uint8_t *W, int64_t row_bytes, const float *grid, int grid_cols,
                         const int8_t *qs, const float *d, float *y, int m, int in_f, int out_f,
                         void *stream);

/*
 * gemv_q8_0_q81_mc, gemv_e4m3_q81_mc, gemv_e4m3_blk128_q81_mc -- the same three products, with
 * the same arguments, checks and return codes, for several activation rows on the matrix
 * cores (v_mfma_i32_16x16x32_i8 for Q8_0, v_mfma_f32_16x16x32_f16 for e4m3): 16 weight rows x
 * up to 8 activation rows per instruction, one q8_1 block (K = 32) at a time.  Opt-in: at
 * m >= 3 the vector kernels of the plain entry points are bound by their per-row arithmetic,
 * not by the weight stream, and these keep the cost nearly flat in m (17408 x 5120: m = 8
 * takes 1.4-1.5x m = 1, against 2.0-2.6x on the vector kernels).
 * What they give up is the bit-parity gate of the batched arms: each block's sum is formed by
 * the matrix core and the block sums are added in a fixed order of their own, so a row agrees
 * with the plain entry point to rounding (within the parity tolerance, 1e-5 of the sum of the
 * terms' magnitudes), not bit for bit.  A row is bit-identical to the same row in any other
 * call of the same entry point, whatever m, its position and the other rows.
 * Row layouts the matrix-core kernels do not take run the plain entry point's kernels: a
 * row_bytes above 64 MiB, and for Q8_0 anything off its fast path (in_f % 256 != 0, W or
 * row_bytes not 16-byte aligned).
 */
int gemv_q8_0_q81_mc(const void *W, int64_t row_bytes, const int8_t *qs, const float *d,
                     float *y, int m, int in_f, int out_f, void *stream);
int gemv_e4m3_q81_mc(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                     const float *d, float *y, int m, int in_f, int out_f, void *stream);
int gemv_e4m3_blk128_q81_mc(const uint8_t *W, int64_t row_bytes, const float *grid,
                            int grid_cols, const int8_t *qs, const float *d, float *y, int m,
                            int in_f, int out_f, void *stream);

/*
 * requant_e4m3_q8_0 -- load-time requantisation of a raw e4m3 weight plane (per-tensor scale)
 * into ggml Q8_0 rows, the container gemv_q8_0_q81 reads.
 * Source: gemv_e4m3_bench.rs, module doc QUESTION (the ship path dequantises FP8 checkpoints
 * to a Q8_0 slab at load).  The page gives no formula; the rule is the 32-value block rule of
 * quantize_q8_1 (q8_fuse_gate.rs, the `id = 1/d` branch) with the scale stored as fp16.  Per
 * 32-block b of row r, every step in f32:
 *   v_i = e4m3(W[r, 32b + i]) * scale,  d = max|v_i| / 127,  id = 1 / d (0 when d == 0),
 *   q_i = round(v_i * id) with halves away from zero,
 *   Wq[r] bytes 34b .. 34b+33 = binary16(d) (round to nearest even, little-endian), q_0..q_31.
 *   W            u8 [out_f] rows of row_bytes bytes (first in_f used); 16-byte aligned,
 *                row_bytes >= in_f and a multiple of 16
 *   scale        finite, and 0 or of magnitude at least 2^-112 (documented, not checked: below
 *                that a block's d can be so small that 1 / d overflows, and its bytes are then
 *                unspecified)
 *   Wq           output rows of q_row_bytes bytes: only the first in_f / 32 * 34 bytes of each
 *                row are written; 2-byte aligned, q_row_bytes >= in_f / 32 * 34 and even; must
 *                not overlap W.  Packed rows (q_row_bytes = in_f / 32 * 34) in a 16-byte
 *                aligned Wq are the fastest layout; with in_f % 256 == 0 they are also the
 *                layout the fast GEMV path needs.
 *   in_f         multiple of 32, <= FP8GEMV_MAX_IN_F;  out_f >= 1
 */
int requant_e4m3_q8_0(const uint8_t *W, int64_t row_bytes, float scale, void *Wq,
                      int64_t q_row_bytes, int in_f, int out_f, void *stream);

/*
 * requant_e4m3_blk128_q8_0 -- the same for a block-128 scaled plane: the block's S is
 * grid[r / 128, b / 4] (each 32-block lies in one 128-column tile).
 * Source: as above, plus THE BLOCK-128 ARM (the f32 [ceil(out_f/128), ceil(in_f/128)] grid).
 *   grid       f32 [ceil(out_f/128), grid_cols], row-major; every value obeys the rule for
 *              scale above; 4-byte aligned
 *   grid_cols  must equal ceil(in_f / 128)
 *   other arguments as for requant_e4m3_q8_0
 */
int requant_e4m3_blk128_q8_0(const uint8_t *W, int64_t row_bytes, const float *grid,
                             int grid_cols, void *Wq, int64_t q_row_bytes, int in_f, int out_f,
                             void *stream);

/*
 * fp8gemv_read_bytes -- measurement aid, not a step of the matvec: streams `bytes` bytes from
 * p with the GEMVs' load pattern (16-byte non-temporal loads, 1 KiB per wave-wide load,
 * 8 KiB per wave, 4-wave workgroups) and discards them; `sink` (one uint32) is written only in
 * the practically impossible case that the folded data equal a fixed constant.  Timing it on
 * a cold range gives the achievable read ceiling the GEMV timings are compared with.  The
 * same as fp8gemv_read_pattern with FP8GEMV_READ_CHUNK8K.
 *   p      device pointer, 16-byte aligned;  1 <= bytes <= FP8GEMV_MAX_READ_BYTES
 *   sink   device pointer to one uint32, 4-byte aligned
 */
#define FP8GEMV_MAX_READ_BYTES ((int64_t)1 << 35)
int fp8gemv_read_bytes(const void *p, int64_t bytes, uint32_t *sink, void *stream);

/*
 * fp8gemv_read_pattern -- measurement aid: the same kind of discarding stream in one of several
 * load patterns, so that the read ceiling is not only the GEMVs' own pattern measured against
 * itself, and so that a launch's fixed cost can be taken apart.  Source of the discipline:
 * gemv_e4m3_bench.rs, DRAM-COLD DISCIPLINE (times are only meaningful on weights that come from
 * DRAM, not from the last-level cache).  Patterns:
 *   FP8GEMV_READ_CHUNK8K     4-wave workgroups, 8 KiB contiguous per wave (8 loads in flight
 *                            per lane), one workgroup per 32 KiB (= fp8gemv_read_bytes)
 *   FP8GEMV_READ_CHUNK16K    as CHUNK8K with 16 KiB per wave (16 loads in flight per lane)
 *   FP8GEMV_READ_WG8         8-wave workgroups, 8 KiB per wave
 *   FP8GEMV_READ_WG16        16-wave workgroups, 8 KiB per wave
 *   FP8GEMV_READ_PERSISTENT  a grid of the device's resident waves (8 four-wave workgroups
 *                            per compute unit); each wave strides over 4 KiB blocks with the
 *                            next block in flight while the current one is folded
 *   FP8GEMV_READ_CACHED      as CHUNK8K without the non-temporal hint
 *   FP8GEMV_READ_ROWS_1K     rows of row_bytes, one wave per row, 1 KiB windows in batches
 *                            of 4 with the next batch in flight (the e4m3 GEMV's m = 1 pattern)
 *   FP8GEMV_READ_ROWS_816    the same with 816-byte windows read by 51 lanes (the Q8_0 GEMV's
 *                            pattern: three 272-byte groups of eight 34-byte blocks)
 *   FP8GEMV_READ_ROWS_ALIGNED  rows of row_bytes, one wave per row, each row read from the
 *                            128-byte line boundary at or before its start in 1 KiB windows
 *                            (whole lines per wave-wide load), batches of 3
 *   FP8GEMV_READ_LINE_WINDOWS  4-wave workgroups each read R consecutive rows (the smallest R
 *                            with R * row_bytes a multiple of 2176) as one span of 2176-byte
 *                            windows (17 whole lines; 8 groups of Q8_0 blocks), window K by
 *                            wave K % 4 as two 1 KiB loads and one 128-byte line, batches of 2
 *   FP8GEMV_READ_EMPTY       CHUNK8K's grid with no loads: dispatch and drain alone
 *   FP8GEMV_READ_ONE_WAVE    one wave loads the first min(bytes, 1 KiB): a launch plus one cold
 *                            round trip to HBM
 *   p, bytes, sink   as for fp8gemv_read_bytes
 *   row_bytes        ROWS_* and LINE_WINDOWS only: 1024 <= row_bytes <= 2^20, a multiple of
 *                    16, and bytes a multiple of it; ignored by the other patterns
 * Returns FP8GEMV_ERR_SHAPE for an unknown pattern or a bad row_bytes.
 */
#define FP8GEMV_READ_CHUNK8K     0
#define FP8GEMV_READ_CHUNK16K    1
#define FP8GEMV_READ_WG8         2
#define FP8GEMV_READ_WG16        3
#define FP8GEMV_READ_PERSISTENT  4
#define FP8GEMV_READ_CACHED      5
#define FP8GEMV_READ_ROWS_1K     6
#define FP8GEMV_READ_ROWS_816    7
#define FP8GEMV_READ_EMPTY       8
#define FP8GEMV_READ_ONE_WAVE    9
#define FP8GEMV_READ_ROWS_ALIGNED 10
#define FP8GEMV_READ_LINE_WINDOWS 11
#define FP8GEMV_READ_NUM_PATTERNS 12
int fp8gemv_read_pattern(const void *p, int64_t bytes, int pattern, int64_t row_bytes,
                         uint32_t *sink, void *stream);

/*
 * fp8gemv_gemv_launch_info -- what one GEMV call with these arguments would launch, without
 * launching it: for profilers and benches that label kernel traces.  The library's own launch
 * selection fills it in, so it always agrees with the launch.
 *   container   FP8GEMV_Q8_0, FP8GEMV_E4M3 or FP8GEMV_E4M3_BLK128 (the plain entry points), or
 *               FP8GEMV_Q8_0_MC, FP8GEMV_E4M3_MC or FP8GEMV_E4M3_BLK128_MC (the *_mc ones)
 *   W, row_bytes, m, in_f, out_f   as for that container's GEMV; W is never dereferenced (only
 *               its alignment matters, for the Q8_0 fast-path choice)
 *   info        out: grid in workgroups (x = weight rows, y = activation-row passes), threads per
 *               workgroup, dynamic LDS bytes, the kernel family and its launch configuration as
 *               they appear in the demangled kernel symbol (static strings).  The launches for
 *               3 or more activation rows on the vector kernels (rows of up to 18432 columns
 *               for e4m3, 24576 for Q8_0) are persistent: their grid_x is the
 *               workgroups that fit on the current device at once (its CU count, read once per
 *               device; 256 CUs are assumed where it cannot be read), whose waves loop over the
 *               weight rows.
 * Returns the argument checks of the GEMV (FP8GEMV_ERR_* as above, W and info must be
 * non-NULL) and FP8GEMV_ERR_SHAPE for an unknown container; reads the current device's CU
 * count at most once, and touches no device memory.
 */
#define FP8GEMV_Q8_0         0
#define FP8GEMV_E4M3         1
#define FP8GEMV_E4M3_BLK128  2
#define FP8GEMV_Q8_0_MC      3
#define FP8GEMV_E4M3_MC      4
#define FP8GEMV_E4M3_BLK128_MC 5
typedef struct {
  uint32_t grid_x, grid_y;
  uint32_t workgroup_size;
  uint32_t lds_bytes;
  const char *kernel;
  const char *config;
} fp8gemv_launch_info;
int fp8gemv_gemv_launch_info(int container, const void *W, int64_t row_bytes, int m, int in_f,
                             int out_f, fp8gemv_launch_info *info);

/* Human-readable text for a return code (static storage, never NULL). */
const char *fp8gemv_strerror(int rc);

#ifdef __cplusplus
}
#endif

#endif /* FP8_GEMV_H */
