/*
 * oracle.cpp -- plain single-threaded CPU reference of one rank's sharded
 * mixed-precision AdamW step over a FlatParameter.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
 * shares no source with the GPU library.  Build: g++ -O2 -ffp-contract=off
 * -fno-fast-math (oracle/build.py); every float expression below is then a
 * sequence of separately rounded IEEE-754 binary32/binary64 operations.
 *
 * Page tags used in the citations:
 *   [DS]  "DeepSpeed 与 FSDP" (docs.ifdog.com)
 *   [SRC] "PyTorch FSDP（Fully Sharded Data Parallel）源码级深度解析" (tbr8.org)
 *   [RD]  ZeRO paper reading, 2kiu.com/news/5312103
 */
#include "oracle.h"

#include <cmath>
#include <cstring>

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t b; std::memcpy(&b, &x, 4); return b; }
static float bits_f32(uint32_t b) { float x; std::memcpy(&x, &b, 4); return x; }

/* Round a binary32 value to a binary format with `prec` significand bits
 * (implicit bit included), minimum normal exponent `emin` and maximum
 * exponent `emax` (bias = emax), `ebits` exponent bits; returns the encoding.
 * This is the IEEE-754 definition of round-to-nearest, ties-to-even, written
 * on integers: |x| = M * 2^E exactly, the target quantum is
 * 2^(max(floor(log2|x|), emin) - prec + 1), and the rounded multiple of that
 * quantum is formed with an explicit remainder test. */
static uint32_t round_to_format(float x, int prec, int emin, int emax, int ebits) {
    const int total_bits = 1 + ebits + (prec - 1);
    const uint32_t sign = (f32_bits(x) >> 31) << (total_bits - 1);
    const uint32_t exp_all_ones = (1u << ebits) - 1u;
    const uint32_t b = f32_bits(x);
    const uint32_t fexp = (b >> 23) & 0xffu;
    const uint32_t fman = b & 0x7fffffu;
    if (fexp == 0xffu) {
        if (fman != 0) /* NaN -> canonical quiet NaN */
            return sign | (exp_all_ones << (prec - 1)) | (1u << (prec - 2));
        return sign | (exp_all_ones << (prec - 1)); /* infinity */
    }
    if (fexp == 0 && fman == 0) return sign; /* signed zero */

    /* |x| = M * 2^E with M an integer */
    uint64_t M;
    int E;
    if (fexp == 0) { M = fman; E = -149; }
    else { M = (uint64_t)(fman | 0x800000u); E = (int)fexp - 150; }
    int msb = 63;
    while (((M >> msb) & 1u) == 0) --msb;
    const int e = msb + E;                         /* floor(log2 |x|) */
    const int qe = (e > emin ? e : emin) - (prec - 1); /* quantum exponent */

    uint64_t n; /* |x| / 2^qe rounded to nearest, ties to even */
    if (E >= qe) {
        n = M << (E - qe);
    } else {
        const int s = qe - E;
        if (s > 60) {
            n = 0; /* far below half a quantum */
        } else {
            n = M >> s;
            const uint64_t rem = M & ((1ull << s) - 1ull);
            const uint64_t half = 1ull << (s - 1);
            if (rem > half || (rem == half && (n & 1ull))) n += 1;
        }
    }
    int q = qe;
    if (n == (1ull << prec)) { n >>= 1; q += 1; } /* carry into next binade */
    /* largest finite value is (2^prec - 1) * 2^(emax - prec + 1) */
    if (q > emax - prec + 1) return sign | (exp_all_ones << (prec - 1));
    if (n < (1ull << (prec - 1))) /* subnormal (or zero) in the target */
        return sign | (uint32_t)n;
    const uint32_t efield = (uint32_t)(q + (prec - 1) + emax);
    const uint32_t mfield = (uint32_t)(n - (1ull << (prec - 1)));
    return sign | (efield << (prec - 1)) | mfield;
}

/* binary16: 11-bit significand, exponents -14..15 (bias 15). */
uint16_t oracle_f32_to_f16(float x) { return (uint16_t)round_to_format(x, 11, -14, 15, 5); }
/* bfloat16: 8-bit significand, exponents -126..127 (bias 127). */
uint16_t oracle_f32_to_bf16(float x) { return (uint16_t)round_to_format(x, 8, -126, 127, 8); }

float oracle_f16_to_f32(uint16_t h) {
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int m = h & 1023;
    double v;
    if (e == 31) {
        if (m != 0) return bits_f32(((uint32_t)s << 31) | 0x7fc00000u);
        v = INFINITY;
    } else if (e == 0) {
        v = std::ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    } else {
        v = std::ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return (float)(s ? -v : v); /* exact: every binary16 value is a binary32 value */
}

/* bfloat16 is by definition the upper half of a binary32 encoding. */
float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

void oracle_f32_to_f16_n(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(x[i]);
}
void oracle_f32_to_bf16_n(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}
void oracle_f16_to_f32_n(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}
void oracle_bf16_to_f32_n(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(h[i]);
}

/* value of element i of a buffer of the given encoding, as binary32 */
static float load_elem(const void* buf, int32_t dtype, int64_t i) {
    if (dtype == OR_F32) return ((const float*)buf)[i];
    if (dtype == OR_F16) return oracle_f16_to_f32(((const uint16_t*)buf)[i]);
    return oracle_bf16_to_f32(((const uint16_t*)buf)[i]);
}
static void store_lp(void* buf, int32_t dtype, int64_t i, float x) {
    if (dtype == OR_F16) ((uint16_t*)buf)[i] = oracle_f32_to_f16(x);
    else ((uint16_t*)buf)[i] = oracle_f32_to_bf16(x);
}

/* ------------------------------------------------------------------------ */
/* FlatParameter layout.                                                     */
/* [SRC] §3.1: parameters are concatenated in order into one 1-D buffer and  */
/* each records its [start, end) offset, with no gap between parameters.     */
/* [DS] "FSDP 的分片粒度与 FlatParameter": each rank owns 1/N of the flat    */
/* buffer.  Reading: equal shards of ceil(T/N) elements (rounded up to       */
/* `align`), the remainder being zero padding at the flat tail, which is     */
/* the only rule under which every rank's Reduce-Scatter output has the     */
/* same size ([SRC] §3.3).                                                   */
/* ------------------------------------------------------------------------ */
int64_t oracle_layout(const int64_t* numels, int32_t n_params, int32_t n_ranks,
                      int64_t align, int64_t out[4], int64_t* starts, int64_t* ends,
                      int32_t rank, int64_t* seg_param, int64_t* seg_off_in_param,
                      int64_t* seg_off_in_shard, int64_t* seg_len, int64_t cap) {
    if (n_params < 0 || n_ranks < 1 || align < 1 || rank < 0 || rank >= n_ranks) return -1;
    int64_t total = 0;
    for (int32_t j = 0; j < n_params; ++j) {
        if (numels[j] < 0) return -1;
        if (starts) starts[j] = total;
        total += numels[j];
        if (ends) ends[j] = total;
    }
    int64_t shard = total / n_ranks + (total % n_ranks != 0 ? 1 : 0); /* ceil(T/N) */
    if (shard % align != 0) shard += align - shard % align;
    const int64_t padded = shard * n_ranks;
    out[0] = total; out[1] = shard; out[2] = padded; out[3] = padded - total;

    const int64_t lo_r = (int64_t)rank * shard, hi_r = lo_r + shard;
    int64_t count = 0, needed = 0;
    int64_t start = 0;
    for (int32_t j = 0; j <= n_params; ++j) {
        int64_t s, e;
        if (j < n_params) { s = start; e = start + numels[j]; start = e; }
        else { s = total; e = padded; } /* tail padding */
        const int64_t lo = s > lo_r ? s : lo_r;
        const int64_t hi = e < hi_r ? e : hi_r;
        if (lo >= hi) continue;
        if (count < cap) {
            seg_param[count] = j < n_params ? j : -1;
            seg_off_in_param[count] = lo - s;
            seg_off_in_shard[count] = lo - lo_r;
            seg_len[count] = hi - lo;
            ++count;
        }
        ++needed;
    }
    if (needed > cap) return -needed - 2;
    return count;
}

/* [DS] "逐步推导" and "ZeRO-3 的数学总结": per-rank bytes are
 *   DP: (P+G+K) Psi;  ZeRO-1: P Psi + G Psi + K Psi/N;
 *   ZeRO-2: P Psi + (G+K) Psi/N;  ZeRO-3: (P+G+K) Psi/N,
 * with Psi/N realised as the padded shard S. */
void oracle_accounting(int64_t total, int64_t shard, int32_t P, int32_t G, int32_t K,
                       int64_t out[4]) {
    out[0] = (int64_t)(P + G + K) * total;
    out[1] = (int64_t)P * total + (int64_t)G * total + (int64_t)K * shard;
    out[2] = (int64_t)P * total + (int64_t)G * shard + (int64_t)K * shard;
    out[3] = (int64_t)P * shard + (int64_t)G * shard + (int64_t)K * shard;
}

/* ------------------------------------------------------------------------ */
/* Reduce half of Reduce-Scatter.                                            */
/* [DS] "ZeRO-2" and the numpy simulation: sum every rank's gradient, then  */
/* keep this rank's slice; [SRC] §3.3: op AVG or SUM; [DS] "实践要点": the  */
/* reduction runs in fp32.  Accumulation is in rank order.                  */
/* ------------------------------------------------------------------------ */
void oracle_reduce(const void* const* bufs, int32_t n_ranks, int32_t dtype, int64_t offset,
                   int64_t n, int32_t op, float* red) {
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t k = 0; k < n_ranks; ++k) acc = acc + load_elem(bufs[k], dtype, offset + i);
        red[i] = (op == OR_AVG) ? acc / (float)n_ranks : acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Gradient accumulation in the sharded state.                               */
/* [DS] "实践要点" (gradient accumulation): a large batch is split into      */
/* micro-batches whose gradients are summed before one optimizer step, the  */
/* loss being divided by the number of micro-steps; [RD] §5.3: under ZeRO   */
/* the gradients are accumulated while sharded; [RD] §5.1 configures two    */
/* accumulation steps.  Reading: every micro-step reduces its N rank        */
/* buffers exactly as oracle_reduce does (the Reduce-Scatter output of that */
/* micro-step), then adds that result to the rank's fp32 shard:             */
/*   acc[i] = acc[i] + red_i.  The 1/steps factor is already in the         */
/* gradients (it is applied to the loss before backward).                   */
/* ------------------------------------------------------------------------ */
void oracle_reduce_accumulate(const void* const* bufs, int32_t n_ranks, int32_t dtype,
                              int64_t offset, int64_t n, int32_t op, float* acc) {
    for (int64_t i = 0; i < n; ++i) {
        float red;
        oracle_reduce(bufs, n_ranks, dtype, offset + i, 1, op, &red);
        acc[i] = acc[i] + red;
    }
}

/* ------------------------------------------------------------------------ */
/* Quantised gradient reduce.                                                */
/* [DS] "ZeRO++：量化通信压缩": gradients travel through the Reduce-Scatter */
/* in a quantised form (its QG scheme), cutting that collective's volume.   */
/* The page gives no scheme; reading: every rank sends its slice for this   */
/* rank as INT8 codes with one fp32 scale per block (the parameter          */
/* payload's scheme, blocks restarting at the slice start), and this rank   */
/* dequantises each rank's value, f32(q) * scale (one binary32 product),    */
/* and sums them in rank order in fp32; AVG divides the sum by N.           */
/* ------------------------------------------------------------------------ */
void oracle_reduce_q8(const int8_t* const* q, const float* const* scales, int32_t n_ranks,
                      int64_t n, int32_t block, int32_t op, float* red) {
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t k = 0; k < n_ranks; ++k) {
            const float x = (float)q[k][i] * scales[k][i / block];
            acc = acc + x;
        }
        red[i] = (op == OR_AVG) ? acc / (float)n_ranks : acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Unscale, overflow test, local sum of squares.                             */
/* [RD] §5.1 (fp16 loss scaling, initial scale 2^16) and §5.3 (overflow is  */
/* detected on the gradients; clipping uses the global gradient norm).      */
/* The gradient is divided by the loss scale, done as a product with the    */
/* exact reciprocal of the (power-of-two) scale.                            */
/* ------------------------------------------------------------------------ */
void oracle_unscale_stats(const void* g, int32_t dtype, int64_t n, float loss_scale,
                          double* sumsq, int32_t* overflow) {
    const float inv = (float)(1.0 / (double)loss_scale);
    double s = *sumsq;
    int32_t ovf = *overflow;
    for (int64_t i = 0; i < n; ++i) {
        const float u = load_elem(g, dtype, i) * inv;
        if (!std::isfinite(u)) ovf = 1;
        s = s + (double)u * (double)u;
    }
    *sumsq = s;
    *overflow = ovf;
}

/* [RD] §5.1 "gradient_clipping: 1.0": scale every gradient by
 * min(1, max_norm / (||g|| + 1e-6)), ||g|| the global L2 norm. */
float oracle_clip_coef(double sumsq_total, double max_norm) {
    if (!(max_norm > 0.0)) return 1.0f;
    const double c = max_norm / (std::sqrt(sumsq_total) + 1e-6);
    return (float)(c < 1.0 ? c : 1.0);
}

/* ------------------------------------------------------------------------ */
/* AdamW on the fp32 master shard, with fp16/bf16 write-back.                */
/* [DS] "ZeRO-Offload" gives Adam with bias correction:                      */
/*   m_t = b1 m + (1-b1) g;  v_t = b2 v + (1-b2) g^2;                         */
/*   mh = m_t/(1-b1^t);  vh = v_t/(1-b2^t);  theta -= lr * mh/(sqrt(vh)+eps) */
/* [RD] §5.1 names AdamW with weight_decay 0.01; decoupled decay multiplies  */
/* theta_{t-1} by (1 - lr*wd).  [SRC] §7.2: the update runs in fp32 on the  */
/* master copy; the fp16/bf16 copy is what the All-Gather sends.            */
/* Scalars are formed in double and rounded once to float; b^t is t         */
/* successive double products.  Per element every operation is one         */
/* rounded binary32 operation, in the order written.                        */
/* ------------------------------------------------------------------------ */
void oracle_adamw(const void* g, int32_t gdtype, float* p, float* m, float* v, int64_t n,
                  float loss_scale, float coef, int64_t t, const oracle_hparams* hp,
                  void* lp_out, int32_t lp_dtype) {
    double pw1 = 1.0, pw2 = 1.0;
    for (int64_t k = 0; k < t; ++k) { pw1 = pw1 * hp->beta1; pw2 = pw2 * hp->beta2; }
    const float b1 = (float)hp->beta1;
    const float c1 = (float)(1.0 - hp->beta1);
    const float b2 = (float)hp->beta2;
    const float c2 = (float)(1.0 - hp->beta2);
    const float bc1 = (float)(1.0 - pw1);
    const float bc2 = (float)(1.0 - pw2);
    const float lr = (float)hp->lr;
    const float wdf = (float)(1.0 - hp->lr * hp->weight_decay);
    const float eps = (float)hp->eps;
    const float inv = (float)(1.0 / (double)loss_scale);
    for (int64_t i = 0; i < n; ++i) {
        const float u = load_elem(g, gdtype, i) * inv; /* unscaled gradient */
        const float gg = u * coef;                     /* clipped gradient */
        const float mn = b1 * m[i] + c1 * gg;
        const float vn = b2 * v[i] + c2 * (gg * gg);
        const float mh = mn / bc1;
        const float vh = vn / bc2;
        const float d = std::sqrt(vh) + eps;
        const float pn = p[i] * wdf - (lr * mh) / d;
        m[i] = mn;
        v[i] = vn;
        p[i] = pn;
        if (lp_out) store_lp(lp_out, lp_dtype, i, pn);
    }
}

/* ------------------------------------------------------------------------ */
/* Blockwise INT8 of the written fp16/bf16 shard.                            */
/* [DS] "ZeRO++": parameter shards are quantised to int8/int4 before the     */
/* All-Gather and dequantised on receipt; [RD] §4.2: the 2-byte payload is  */
/* cut to INT8.  The pages fix no scheme; reading: symmetric absmax per     */
/* block, scale = amax/127, codes rint(x/scale) clamped to [-127, 127].     */
/* ------------------------------------------------------------------------ */
void oracle_quant_int8(const void* x, int32_t dtype, int64_t n, int32_t block, int8_t* q,
                       float* scales) {
    const int64_t nb = (n + block - 1) / block;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * block;
        const int64_t hi = lo + block < n ? lo + block : n;
        float amax = 0.0f;
        for (int64_t j = lo; j < hi; ++j) {
            const float a = std::fabs(load_elem(x, dtype, j));
            if (a > amax) amax = a;
        }
        const float scale = amax / 127.0f;
        scales[b] = scale;
        for (int64_t j = lo; j < hi; ++j) {
            if (amax == 0.0f) { q[j] = 0; continue; }
            float r = std::nearbyint(load_elem(x, dtype, j) / scale); /* ties to even */
            if (std::isnan(r)) r = 0.0f;
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[j] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* INT8 All-Gather consumer.                                                 */
/* [DS] "ZeRO++：量化通信压缩": the receiver dequantises the int8/int4       */
/* parameter shards it gathers; [RD] §4.2: the INT8 weights are restored    */
/* only just before local compute; [DS] "FSDP 的分片粒度与 FlatParameter":  */
/* the gathered flat buffer is then unflattened into the parameters (views  */
/* at each parameter's [start, end) flat range, no arithmetic).             */
/* The gathered payload holds n_slots rank slots: slot s's codes at         */
/* q[s*S .. s*S+S) and its scales at scales[s*nb ..), nb = ceil(S/block),   */
/* blocks restarting at each slot's start (as the producer wrote them).     */
/* Reading: x = f32(q) * scale, one binary32 product, then rounded to the   */
/* parameter format (RNE); out[s*S + i] in the full flat buffer.            */
/* ------------------------------------------------------------------------ */
void oracle_dequant_int8(const int8_t* q, const float* scales, int32_t n_slots,
                         int64_t slot_numel, int32_t block, int32_t dtype, void* out) {
    const int64_t nb = (slot_numel + block - 1) / block;
    for (int32_t s = 0; s < n_slots; ++s) {
        for (int64_t i = 0; i < slot_numel; ++i) {
            const int64_t j = (int64_t)s * slot_numel + i;
            const float x = (float)q[j] * scales[(int64_t)s * nb + i / block];
            if (dtype == OR_F32) static_cast<float*>(out)[j] = x;
            else store_lp(out, dtype, j, x);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Loss scaler.  [RD] §5.1: dynamic scale ("loss_scale": 0) starting at      */
/* 2^16 with a window of 1000; §5.3: the scale shrinks on overflow and grows */
/* after a stretch without one, and an overflow step is not applied.        */
/* Reading: halve (not below min_scale) on overflow, double after `window`  */
/* consecutive good steps.                                                   */
/* ------------------------------------------------------------------------ */
void oracle_scaler_update(oracle_scaler* s, int32_t overflow) {
    if (overflow) {
        if (s->dynamic) {
            const float h = s->loss_scale / 2.0f;
            s->loss_scale = h > s->min_scale ? h : s->min_scale;
        }
        s->good_steps = 0;
        return;
    }
    s->step += 1;
    if (s->dynamic) {
        s->good_steps += 1;
        if (s->good_steps == s->window) {
            /* doubling stops at 2^127, the largest binary32 power of two */
            if (s->loss_scale < 0x1p127f) s->loss_scale = s->loss_scale * 2.0f;
            s->good_steps = 0;
        }
    }
}
