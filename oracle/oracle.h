/*
 * oracle.h -- CPU reference ("oracle") for one rank's sharded mixed-precision
 * AdamW step over a FlatParameter.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that tests, the smoke
 * check and the benchmark's CPU-baseline leg can compare the GPU library
 * against a plain, slow, obviously correct statement of what the step
 * computes.  Nothing on the product path may link, load or call it.  It shares
 * no source with the GPU library (its own types, its own fp16/bf16
 * converters, its own layout arithmetic) and is compiled by g++ with
 * contraction off (no FMA) and no fast-math, so every float operation below
 * is one IEEE-754 operation, rounded to nearest-even.
 *
 * Sources (three web pages; cited by title and section):
 *   [DS]  "DeepSpeed 与 FSDP" (docs.ifdog.com, foundations/04-training)
 *   [SRC] "PyTorch FSDP（Fully Sharded Data Parallel）源码级深度解析" (tbr8.org)
 *   [RD]  the ZeRO paper reading at 2kiu.com/news/5312103 (its page title
 *         is an unrelated heading; cited by address)
 *
 * Every function is single-threaded and walks its range in index order.
 * Parity of every function here is pinned by tests/test_oracle_*.py against
 * values printed on the pages, closed forms, brute force or exact rational
 * arithmetic; none is "parity unpinned" except where noted below.
 */
#ifndef ZEROFLAT_ORACLE_H
#define ZEROFLAT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element encodings understood by the oracle */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
/* reduction operator of the Reduce-Scatter */
enum { OR_SUM = 0, OR_AVG = 1 };

/* ---- number formats --------------------------------------------------- */
/* IEEE-754 binary16 and bfloat16 <-> binary32, round-to-nearest-even.  NaN
 * maps to the canonical quiet NaN of the target format, sign kept. */
uint16_t oracle_f32_to_f16(float x);
float    oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float x);
float    oracle_bf16_to_f32(uint16_t h);
void oracle_f32_to_f16_n(const float* x, int64_t n, uint16_t* out);
void oracle_f32_to_bf16_n(const float* x, int64_t n, uint16_t* out);
void oracle_f16_to_f32_n(const uint16_t* h, int64_t n, float* out);
void oracle_bf16_to_f32_n(const uint16_t* h, int64_t n, float* out);

/* ---- FlatParameter layout and memory accounting ----------------------- */
/* Fills out[0..3] = {total T, shard S, padded N*S, pad}; starts/ends (may be
 * NULL) get each parameter's [start,end) flat range; for rank `rank` the
 * pieces of that rank's shard are written to seg_* (param index, offset in
 * param, offset in shard, length; param = -1 for tail padding), at most
 * `cap` of them; returns the piece count, or -1 on invalid input, or
 * -(needed) - 2 if cap is too small. */
int64_t oracle_layout(const int64_t* numels, int32_t n_params, int32_t n_ranks,
                      int64_t align, int64_t out[4], int64_t* starts, int64_t* ends,
                      int32_t rank, int64_t* seg_param, int64_t* seg_off_in_param,
                      int64_t* seg_off_in_shard, int64_t* seg_len, int64_t cap);

/* per-rank bytes under pure DP, ZeRO-1, ZeRO-2, ZeRO-3 (out[0..3]) for a
 * model of `total` parameters sharded `shard` per rank, with param_bytes,
 * grad_bytes and optim_bytes per parameter. */
void oracle_accounting(int64_t total, int64_t shard, int32_t param_bytes,
                       int32_t grad_bytes, int32_t optim_bytes, int64_t out[4]);

/* ---- the step ---------------------------------------------------------- */
/* Reduce half of Reduce-Scatter: red[i] = sum_k f32(buf_k[offset+i]) in rank
 * order k = 0..N-1 (fp32 accumulator); AVG divides the sum by N. */
void oracle_reduce(const void* const* bufs, int32_t n_ranks, int32_t dtype,
                   int64_t offset, int64_t n, int32_t op, float* red);

/* Gradient accumulation in the sharded state: acc[i] = acc[i] + red_i, with
 * red_i exactly oracle_reduce's value for this micro-step's buffers. */
void oracle_reduce_accumulate(const void* const* bufs, int32_t n_ranks, int32_t dtype,
                              int64_t offset, int64_t n, int32_t op, float* acc);

/* Quantised gradient reduce: rank k's slice arrives as INT8 codes q[k][0..n)
 * with fp32 scales scales[k][i / block];
 *   red[i] = sum_k f32(q[k][i]) * scales[k][i / block]  (rank order, fp32),
 * AVG divides the sum by N. */
void oracle_reduce_q8(const int8_t* const* q, const float* const* scales, int32_t n_ranks,
                      int64_t n, int32_t block, int32_t op, float* red);

/* Unscale + overflow + local sum of squares over g[0..n):
 *   u_i = f32(g_i) * f32(1/loss_scale); overflow |= !isfinite(u_i);
 *   sumsq += (double)u_i * (double)u_i, in index order. */
void oracle_unscale_stats(const void* g, int32_t dtype, int64_t n, float loss_scale,
                          double* sumsq, int32_t* overflow);

/* Global-norm clip coefficient (float) min(1, max_norm/(sqrt(sumsq)+1e-6));
 * 1 when max_norm <= 0. */
float oracle_clip_coef(double sumsq_total, double max_norm);

typedef struct {
    double lr, beta1, beta2, eps, weight_decay, max_grad_norm;
} oracle_hparams;

/* AdamW (decoupled weight decay) on n elements at step t >= 1.
 *   g input is the reduced gradient (fp32, or fp16/bf16 when pre-reduced),
 *   p, m, v are updated in place, and lp_out (may be NULL) receives the
 *   fp16/bf16 rounding of the new p.  Scalars: see oracle.cpp. */
void oracle_adamw(const void* g, int32_t gdtype, float* p, float* m, float* v, int64_t n,
                  float loss_scale, float coef, int64_t t, const oracle_hparams* hp,
                  void* lp_out, int32_t lp_dtype);

/* Blockwise symmetric INT8 of n fp16/bf16 values: per block of `block`
 * elements (the last may be short) scale = amax/127, q = clamp(rint(x/scale)). */
void oracle_quant_int8(const void* x, int32_t dtype, int64_t n, int32_t block,
                       int8_t* q, float* scales);

/* INT8 All-Gather consumer: n_slots slots of slot_numel codes (scales of
 * slot s at s*ceil(slot_numel/block)) -> out[s*slot_numel + i] =
 * round_dtype(f32(q) * scale); dtype OR_F32, OR_F16 or OR_BF16. */
void oracle_dequant_int8(const int8_t* q, const float* scales, int32_t n_slots,
                         int64_t slot_numel, int32_t block, int32_t dtype, void* out);

/* Dynamic/static loss scaler, applied once per step after the overflow test. */
typedef struct {
    float loss_scale;     /* current scale (a power of two) */
    float min_scale;      /* floor when halving */
    int32_t dynamic;      /* 0 => the scale never changes */
    int32_t window;       /* good steps before the scale doubles */
    int32_t good_steps;   /* consecutive non-overflow steps */
    int32_t step;         /* successful (non-skipped) steps so far */
} oracle_scaler;
void oracle_scaler_update(oracle_scaler* s, int32_t overflow);

#ifdef __cplusplus
}
#endif
#endif
