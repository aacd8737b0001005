// zeroflat_api.cpp -- the extern "C" entry points of libzeroflat: argument
// validation, the FlatParameter layout (host integer arithmetic), the
// host-side scalars of the AdamW step, and dispatch to the gfx950 kernels.
// Nothing here allocates device memory or synchronizes.
#include <math.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "zeroflat.h"
#include "zf_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return ZERO_OK;
}

int hip_fail(int e, const char* where) {
    return fail(ZERO_EHIP, "%s: HIP error %d (%s)", where, e, zf::hip_error_string(e));
}

bool valid_dtype(int32_t d) { return d == ZERO_F32 || d == ZERO_F16 || d == ZERO_BF16; }
int esize(int32_t d) { return d == ZERO_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// the cache line the streaming reads are laid out on
constexpr uintptr_t kLineBytes = 128;

// the device address of the state's per-block partial-sum table (the state
// pointer is a device address: computed, never dereferenced, here)
double* state_partials(zero_step_state_t* st) {
    return st ? reinterpret_cast<double*>(reinterpret_cast<char*>(st) +
                                          offsetof(zero_step_state_t, partials))
              : nullptr;
}

// a*b, false on int64 overflow
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

}  // namespace

extern "C" {

const char* zero_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------------------
// FlatParameter layout ("PyTorch FSDP 源码级深度解析" §3.1 offsets; equal
// padded shards so that every rank's Reduce-Scatter output has one size,
// §3.3) and per-rank accounting ("DeepSpeed 与 FSDP", ZeRO-3 的数学总结).
int zero_flat_layout(const int64_t* numels, int32_t n_params, int32_t n_ranks, int64_t align,
                     int32_t param_bytes, int32_t grad_bytes, int32_t optim_bytes,
                     int32_t rank, zero_layout_t* out, zero_span_t* spans,
                     zero_segment_t* segs, int32_t segs_cap, int32_t* n_segs) {
    if (!out) return fail(ZERO_EINVAL, "zero_flat_layout: out is NULL");
    if (n_params < 0 || (n_params > 0 && !numels))
        return fail(ZERO_EINVAL, "zero_flat_layout: bad parameter list");
    if (n_ranks < 1) return fail(ZERO_EINVAL, "zero_flat_layout: n_ranks must be >= 1");
    if (align < 1) return fail(ZERO_EINVAL, "zero_flat_layout: align must be >= 1");
    if (rank < 0 || rank >= n_ranks) return fail(ZERO_EINVAL, "zero_flat_layout: rank out of range");
    if (param_bytes < 0 || grad_bytes < 0 || optim_bytes < 0)
        return fail(ZERO_EINVAL, "zero_flat_layout: negative byte counts");
    if (segs_cap < 0 || (segs_cap > 0 && !segs))
        return fail(ZERO_EINVAL, "zero_flat_layout: bad segment buffer");

    int64_t total = 0;
    for (int32_t j = 0; j < n_params; ++j) {
        if (numels[j] < 0) return fail(ZERO_EINVAL, "zero_flat_layout: numel[%d] < 0", j);
        if (!add_ok(total, numels[j], &total)) return fail(ZERO_ERANGE, "zero_flat_layout: total overflows");
    }
    // S = ceil(T / N) rounded up to a multiple of align
    int64_t shard = total / n_ranks + (total % n_ranks ? 1 : 0);
    const int64_t rem = shard % align;
    if (rem && !add_ok(shard, align - rem, &shard))
        return fail(ZERO_ERANGE, "zero_flat_layout: shard overflows");
    int64_t padded;
    if (!mul_ok(shard, n_ranks, &padded)) return fail(ZERO_ERANGE, "zero_flat_layout: padded overflows");

    zero_layout_t L;
    memset(&L, 0, sizeof L);
    L.total = total;
    L.shard = shard;
    L.padded = padded;
    L.pad = padded - total;
    L.n_ranks = n_ranks;
    L.align = align;
    const int64_t P = param_bytes, G = grad_bytes, K = optim_bytes;
    int64_t t0 = 0, t1 = 0, t2 = 0;
    bool good = mul_ok(P + G + K, total, &L.bytes_dp);
    good = good && mul_ok(P + G, total, &t0) && mul_ok(K, shard, &t1) && add_ok(t0, t1, &L.bytes_z1);
    good = good && mul_ok(P, total, &t0) && mul_ok(G + K, shard, &t1) && add_ok(t0, t1, &L.bytes_z2);
    good = good && mul_ok(P + G + K, shard, &t2);
    L.bytes_z3 = t2;
    if (!good) return fail(ZERO_ERANGE, "zero_flat_layout: byte accounting overflows");
    *out = L;

    // pieces of rank r's shard [r*S, (r+1)*S): parameters in order, then padding
    const int64_t lo_r = (int64_t)rank * shard, hi_r = lo_r + shard;
    int32_t count = 0;
    int64_t start = 0;
    for (int32_t j = 0; j <= n_params; ++j) {
        const int64_t s = j < n_params ? start : total;
        const int64_t e = j < n_params ? start + numels[j] : padded;
        if (spans && j < n_params) { spans[j].start = s; spans[j].end = e; }
        if (j < n_params) start = e;
        const int64_t lo = s > lo_r ? s : lo_r;
        const int64_t hi = e < hi_r ? e : hi_r;
        if (lo >= hi) continue;
        if (segs && count < segs_cap) {
            segs[count].param = j < n_params ? j : -1;
            segs[count].reserved = 0;
            segs[count].off_in_param = lo - s;
            segs[count].off_in_shard = lo - lo_r;
            segs[count].len = hi - lo;
        }
        ++count;
    }
    if (n_segs) *n_segs = count;
    if (segs && count > segs_cap)
        return fail(ZERO_ERANGE, "zero_flat_layout: %d segments do not fit in %d", count, segs_cap);
    return ok();
}

// ---------------------------------------------------------------------------
int zero_step_state_init(zero_step_state_t* st, float loss_scale, int32_t dynamic, int32_t window,
                         float min_scale) {
    if (!st) return fail(ZERO_EINVAL, "zero_step_state_init: state is NULL");
    if (!(min_scale >= 1.0f)) return fail(ZERO_EINVAL, "zero_step_state_init: min_scale must be >= 1");
    int ex;
    const float mant = frexpf(loss_scale, &ex);
    if (!(loss_scale >= min_scale) || mant != 0.5f || loss_scale > 1e38f)
        return fail(ZERO_EINVAL, "zero_step_state_init: loss_scale must be a power of two >= min_scale");
    if (dynamic && window < 1) return fail(ZERO_EINVAL, "zero_step_state_init: window must be >= 1");
    memset(st, 0, sizeof *st);
    st->loss_scale = loss_scale;
    st->min_scale = min_scale;
    st->dynamic = dynamic ? 1 : 0;
    st->window = window;
    st->beta1_pow = 1.0;
    st->beta2_pow = 1.0;
    return ok();
}

// ---------------------------------------------------------------------------
namespace {
// zero_grad_reduce_shard, zero_grad_accumulate_shard and
// zero_grad_reduce_shard_noalloc: the same reduce, the second adding into its
// output instead of overwriting it, the third keeping the statistics' partial
// sums in the library's device scratch instead of the state.
int reduce_entry(const char* fn, const void* const* grad_bufs, int32_t n_ranks, int32_t in_dtype,
                 int64_t elem_offset, int64_t shard_numel, int32_t op, float* red_out,
                 int accumulate, zero_step_state_t* d_state, void* stream, bool noalloc = false) {
    if (!grad_bufs) return fail(ZERO_EINVAL, "%s: grad_bufs is NULL", fn);
    if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
        return fail(ZERO_ERANGE, "%s: n_ranks %d not in [1, %d]", fn, n_ranks, ZERO_MAX_RANKS);
    if (!valid_dtype(in_dtype)) return fail(ZERO_EINVAL, "%s: bad in_dtype %d", fn, in_dtype);
    if (op != ZERO_SUM && op != ZERO_AVG) return fail(ZERO_EINVAL, "%s: bad op %d", fn, op);
    if (elem_offset < 0 || shard_numel < 0)
        return fail(ZERO_EINVAL, "%s: negative offset or size", fn);
    if (shard_numel == 0) return ok();  // nothing is read or written
    if (!red_out) return fail(ZERO_EINVAL, "%s: output shard is NULL", fn);
    if (!aligned(red_out, 4)) return fail(ZERO_EALIGN, "%s: output shard not 4-byte aligned", fn);
    if (d_state && !aligned(d_state, 8)) return fail(ZERO_EALIGN, "%s: state not 8-byte aligned", fn);
    const int es = esize(in_dtype);
    zf::ReduceLaunch a;
    memset(&a, 0, sizeof a);
    // vector path: each lane reads 4 consecutive inputs (8 B for 16-bit, 16 B
    // for fp32) and writes (and, accumulating, reads) 4 fp32 outputs (16 B).
    // Rank slices that all start at one offset within a quad keep it, wherever
    // they start ("PyTorch FSDP 源码级深度解析" §3.3: rank r's slice starts at
    // r*S, for any S): the elements up to the first slice's next 128-byte line
    // go element-wise, then the tiles read whole lines and their reduced quads
    // are shifted onto the aligned output.
    const uintptr_t quad = 4 * (uintptr_t)es;
    bool vec = aligned(red_out, 16);
    uintptr_t mis = 0, line_off = 0;
    for (int32_t k = 0; k < n_ranks; ++k) {
        if (!grad_bufs[k]) return fail(ZERO_EINVAL, "%s: grad_bufs[%d] is NULL", fn, k);
        if (!aligned(grad_bufs[k], es))
            return fail(ZERO_EALIGN, "%s: grad_bufs[%d] misaligned", fn, k);
        const char* p = static_cast<const char*>(grad_bufs[k]) + elem_offset * es;
        a.bufs[k] = p;
        const uintptr_t m = (uintptr_t)p % quad;
        if (k == 0) {
            mis = m;
            line_off = (uintptr_t)p % kLineBytes;
        }
        vec = vec && m == mis;
    }
    a.n_ranks = n_ranks;
    a.dtype = in_dtype;
    a.op = op;
    a.vec = vec ? 1 : 0;
    a.head = vec && line_off ? (int32_t)((kLineBytes - line_off) / es) : 0;
    a.n = shard_numel;
    a.red_out = red_out;
    a.accumulate = accumulate;
    a.st = d_state;
    a.partials = state_partials(d_state);
    const int e = noalloc ? zf::launch_reduce_noalloc(a, stream) : zf::launch_reduce_stats(a, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}
}  // namespace

int zero_grad_reduce_shard(const void* const* grad_bufs, int32_t n_ranks, int32_t in_dtype,
                           int64_t elem_offset, int64_t shard_numel, int32_t op,
                           float* red_out, zero_step_state_t* d_state, void* stream) {
    return reduce_entry("zero_grad_reduce_shard", grad_bufs, n_ranks, in_dtype, elem_offset,
                        shard_numel, op, red_out, 0, d_state, stream);
}

// The same reduce for callers that cannot allocate: the statistics' partial
// sums go to the library's per-device scratch, so d_state needs only the
// header of zero_step_state_t.
int zero_grad_reduce_shard_noalloc(const void* const* grad_bufs, int32_t n_ranks,
                                   int32_t in_dtype, int64_t elem_offset, int64_t shard_numel,
                                   int32_t op, float* red_out, zero_step_state_t* d_state,
                                   void* stream) {
    return reduce_entry("zero_grad_reduce_shard_noalloc", grad_bufs, n_ranks, in_dtype,
                        elem_offset, shard_numel, op, red_out, 0, d_state, stream, true);
}

// ---------------------------------------------------------------------------
// Gradient accumulation in the sharded state ("DeepSpeed 与 FSDP", 实践要点;
// 2kiu.com §5.3): acc += this micro-step's reduce.
int zero_grad_accumulate_shard(const void* const* grad_bufs, int32_t n_ranks, int32_t in_dtype,
                               int64_t elem_offset, int64_t shard_numel, int32_t op, float* acc,
                               zero_step_state_t* d_state, void* stream) {
    return reduce_entry("zero_grad_accumulate_shard", grad_bufs, n_ranks, in_dtype, elem_offset,
                        shard_numel, op, acc, 1, d_state, stream);
}

int zero_unscale_norm(const void* grad_shard, int32_t dtype, int64_t n, zero_step_state_t* d_state,
                      void* stream) {
    if (!d_state) return fail(ZERO_EINVAL, "zero_unscale_norm: NULL state");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "zero_unscale_norm: bad dtype %d", dtype);
    if (n < 0) return fail(ZERO_EINVAL, "zero_unscale_norm: n < 0");
    if (n == 0) return ok();  // nothing is read
    if (!grad_shard) return fail(ZERO_EINVAL, "zero_unscale_norm: grad_shard is NULL");
    if (!aligned(grad_shard, esize(dtype))) return fail(ZERO_EALIGN, "zero_unscale_norm: grad misaligned");
    if (!aligned(d_state, 8)) return fail(ZERO_EALIGN, "zero_unscale_norm: state not 8-byte aligned");
    zf::ReduceLaunch a;
    memset(&a, 0, sizeof a);
    a.bufs[0] = grad_shard;
    a.n_ranks = 1;
    a.dtype = dtype;
    a.op = ZERO_SUM;
    // the vector path from the shard's first 128-byte line boundary on (the
    // head before it element-wise)
    const uintptr_t line_off = (uintptr_t)grad_shard % kLineBytes;
    a.vec = 1;
    a.head = line_off ? (int32_t)((kLineBytes - line_off) / esize(dtype)) : 0;
    a.n = n;
    a.red_out = nullptr;
    a.st = d_state;
    a.partials = state_partials(d_state);
    const int e = zf::launch_reduce_stats(a, stream);
    if (e) return hip_fail(e, "zero_unscale_norm");
    return ok();
}

// ---------------------------------------------------------------------------
int zero_adamw_shard_step(const void* grad_shard, int32_t grad_dtype, float* master,
                          float* exp_avg, float* exp_avg_sq, int64_t n, void* allgather_buf,
                          int32_t param_dtype, int64_t slot_offset, int8_t* q_buf,
                          float* q_scales, int64_t q_slot_offset, int64_t q_scale_offset,
                          int32_t q_block, const zero_adamw_hparams_t* hp, uint32_t flags,
                          zero_step_state_t* d_state, void* stream) {
    const char* fn = "zero_adamw_shard_step";
    if (!hp || !d_state) return fail(ZERO_EINVAL, "%s: NULL hp or state", fn);
    if (n < 0 || slot_offset < 0) return fail(ZERO_EINVAL, "%s: negative size or offset", fn);
    if (flags & ~ZERO_STEP_FINALIZE) return fail(ZERO_EINVAL, "%s: unknown flags 0x%x", fn, flags);
    if (!valid_dtype(grad_dtype)) return fail(ZERO_EINVAL, "%s: bad grad_dtype %d", fn, grad_dtype);
    if (param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: param_dtype must be fp16 or bf16", fn);
    if (n > 0 && (!grad_shard || !master || !exp_avg || !exp_avg_sq || !allgather_buf))
        return fail(ZERO_EINVAL, "%s: NULL tensor pointer", fn);
    if (!(hp->lr >= 0.0) || !(hp->eps > 0.0) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->weight_decay >= 0.0))
        return fail(ZERO_EINVAL, "%s: hyper-parameters out of range", fn);
    if (!aligned(d_state, 8)) return fail(ZERO_EALIGN, "%s: state not 8-byte aligned", fn);
    const bool quant = q_buf != nullptr;
    if (quant) {
        if (!q_scales) return fail(ZERO_EINVAL, "%s: q_scales is NULL", fn);
        if (q_block != 256) return fail(ZERO_EINVAL, "%s: q_block must be 256", fn);
        if (q_slot_offset < 0 || q_scale_offset < 0) return fail(ZERO_EINVAL, "%s: negative INT8 offset", fn);
        if (!aligned(q_scales, 4)) return fail(ZERO_EALIGN, "%s: q_scales misaligned", fn);
    }
    zf::AdamLaunch a;
    memset(&a, 0, sizeof a);
    const int ges = esize(grad_dtype);
    if (n > 0) {
        if (!aligned(grad_shard, ges) || !aligned(master, 4) || !aligned(exp_avg, 4) ||
            !aligned(exp_avg_sq, 4) || !aligned(allgather_buf, 2))
            return fail(ZERO_EALIGN, "%s: a tensor is not aligned to its element size", fn);
    }
    a.g = grad_shard;
    a.gdtype = grad_dtype;
    a.pdtype = param_dtype;
    a.p = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.n = n;
    a.lp = static_cast<uint16_t*>(allgather_buf) + slot_offset;
    a.q = quant ? q_buf + q_slot_offset : nullptr;
    a.qs = quant ? q_scales + q_scale_offset : nullptr;
    // vector path: 16-byte fp32 quads and grad quads of 4*ges bytes; the slot
    // (8-byte quads) and the INT8 codes (4-byte quads) at any element offset:
    // rank r's slot starts at r*S ("PyTorch FSDP 源码级深度解析" §3.3), and
    // gfx950 carries out a vector store that is not aligned to its size (the
    // slot and codes are 3 of the update's 28-31 bytes per parameter)
    const bool vec = aligned(master, 16) && aligned(exp_avg, 16) && aligned(exp_avg_sq, 16) &&
                     aligned(grad_shard, 4 * ges);
    a.vec = vec ? 1 : 0;
    a.flags = flags;
    // step scalars formed in double and rounded once to fp32
    a.b1 = (float)hp->beta1;
    a.c1 = (float)(1.0 - hp->beta1);
    a.b2 = (float)hp->beta2;
    a.c2 = (float)(1.0 - hp->beta2);
    a.lr = (float)hp->lr;
    a.wdf = (float)(1.0 - hp->lr * hp->weight_decay);
    a.eps = (float)hp->eps;
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.max_norm = hp->max_grad_norm;
    a.st = d_state;
    const int e = zf::launch_adamw(a, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}

// ---------------------------------------------------------------------------
int zero_quant_allgather_slot(const void* slot, int32_t dtype, int64_t n, int32_t block,
                              int8_t* q_buf, int64_t q_slot_offset, float* q_scales,
                              int64_t q_scale_offset, void* stream) {
    const char* fn = "zero_quant_allgather_slot";
    if (dtype != ZERO_F16 && dtype != ZERO_BF16) return fail(ZERO_EINVAL, "%s: dtype must be fp16 or bf16", fn);
    if (block != 256) return fail(ZERO_EINVAL, "%s: block must be 256", fn);
    if (n < 0 || q_slot_offset < 0 || q_scale_offset < 0) return fail(ZERO_EINVAL, "%s: negative size", fn);
    if (n == 0) return ok();
    if (!slot || !q_buf || !q_scales) return fail(ZERO_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(slot, 2) || !aligned(q_scales, 4)) return fail(ZERO_EALIGN, "%s: misaligned", fn);
    zf::QuantLaunch a;
    a.x = slot;
    a.dtype = dtype;
    a.n = n;
    a.q = q_buf + q_slot_offset;
    a.qs = q_scales + q_scale_offset;
    // 2: eight elements per lane (16-byte slot, 8-byte codes); 1: quad tiles
    a.vec = (aligned(slot, 16) && aligned(a.q, 8)) ? 2 : (aligned(slot, 8) && aligned(a.q, 4)) ? 1 : 0;
    const int e = zf::launch_quant(a, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}

// ---------------------------------------------------------------------------
// Quantised gradient reduce ("DeepSpeed 与 FSDP", ZeRO++：量化通信压缩).
int zero_grad_reduce_shard_int8(const int8_t* const* q_bufs, const float* const* scale_bufs,
                                int32_t n_ranks, int64_t shard_numel, int32_t block, int32_t op,
                                float* red_out, zero_step_state_t* d_state, void* stream) {
    const char* fn = "zero_grad_reduce_shard_int8";
    if (!q_bufs || !scale_bufs) return fail(ZERO_EINVAL, "%s: NULL pointer table", fn);
    if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS / 2)
        return fail(ZERO_ERANGE, "%s: n_ranks %d not in [1, %d]", fn, n_ranks, ZERO_MAX_RANKS / 2);
    if (op != ZERO_SUM && op != ZERO_AVG) return fail(ZERO_EINVAL, "%s: bad op %d", fn, op);
    if (shard_numel < 0) return fail(ZERO_EINVAL, "%s: negative size", fn);
    if (block < 4 || block % 4 != 0) return fail(ZERO_EINVAL, "%s: block %d is not a positive multiple of 4", fn, block);
    if (shard_numel == 0) return ok();  // nothing is read or written
    if (!red_out) return fail(ZERO_EINVAL, "%s: red_out is NULL", fn);
    if (!aligned(red_out, 4)) return fail(ZERO_EALIGN, "%s: red_out not 4-byte aligned", fn);
    if (d_state && !aligned(d_state, 8)) return fail(ZERO_EALIGN, "%s: state not 8-byte aligned", fn);
    zf::ReduceLaunch a;
    memset(&a, 0, sizeof a);
    bool vec = aligned(red_out, 16);
    for (int32_t k = 0; k < n_ranks; ++k) {
        if (!q_bufs[k] || !scale_bufs[k]) return fail(ZERO_EINVAL, "%s: rank %d's payload is NULL", fn, k);
        if (!aligned(scale_bufs[k], 4)) return fail(ZERO_EALIGN, "%s: scale_bufs[%d] misaligned", fn, k);
        a.bufs[2 * k] = q_bufs[k];
        a.bufs[2 * k + 1] = scale_bufs[k];
        vec = vec && aligned(q_bufs[k], 4);
    }
    a.n_ranks = n_ranks;
    a.dtype = ZERO_F32;  // unused by the INT8 source
    a.op = op;
    a.vec = vec ? 1 : 0;
    a.n = shard_numel;
    a.red_out = red_out;
    a.block = block;
    a.block_shift = (block & (block - 1)) == 0 ? __builtin_ctz((unsigned)block) : -1;
    a.st = d_state;
    a.partials = state_partials(d_state);
    const int e = zf::launch_reduce_q8(a, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}

// ---------------------------------------------------------------------------
// ZeRO-Offload ("DeepSpeed 与 FSDP", ZeRO-Offload; 2kiu.com §4.1, §5.1).
namespace {
int check_hp(const char* fn, const zero_adamw_hparams_t* hp) {
    if (!hp) return fail(ZERO_EINVAL, "%s: NULL hp", fn);
    if (!(hp->lr >= 0.0) || !(hp->eps > 0.0) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->weight_decay >= 0.0))
        return fail(ZERO_EINVAL, "%s: hyper-parameters out of range", fn);
    return ZERO_OK;
}
}  // namespace

namespace {
// The gradient array and the 16-bit parameter array of the host step: either
// disjoint, or the very same array when the gradient is 16-bit too (in-place
// staging, each element's gradient read before its parameter is stored).
bool staging_ok(const void* g, int gsize, const void* lp, int64_t n) {
    if (g == lp) return gsize == 2;
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(g), g1 = g0 + (uintptr_t)n * gsize;
    const uintptr_t l0 = reinterpret_cast<uintptr_t>(lp), l1 = l0 + (uintptr_t)n * 2;
    return g1 <= l0 || l1 <= g0;
}
}  // namespace

int zero_offload_adamw_host(const void* grad, int32_t grad_dtype, float* master, float* exp_avg,
                            float* exp_avg_sq, int64_t n, void* lp_out, int32_t param_dtype,
                            const zero_adamw_hparams_t* hp, const zero_step_state_t* host_state,
                            int32_t n_threads, int32_t* skipped) {
    const char* fn = "zero_offload_adamw_host";
    if (int e = check_hp(fn, hp)) return e;
    if (!host_state || !skipped) return fail(ZERO_EINVAL, "%s: NULL state or skipped", fn);
    if (!valid_dtype(grad_dtype)) return fail(ZERO_EINVAL, "%s: bad grad_dtype %d", fn, grad_dtype);
    if (param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: param_dtype must be fp16 or bf16", fn);
    if (n < 0 || n_threads < 0) return fail(ZERO_EINVAL, "%s: negative size or thread count", fn);
    if (n > 0 && (!grad || !master || !exp_avg || !exp_avg_sq || !lp_out))
        return fail(ZERO_EINVAL, "%s: NULL array", fn);
    if (n > 0 && (!aligned(grad, esize(grad_dtype)) || !aligned(master, 4) || !aligned(exp_avg, 4) ||
                  !aligned(exp_avg_sq, 4) || !aligned(lp_out, 2)))
        return fail(ZERO_EALIGN, "%s: an array is not aligned to its element size", fn);
    if (n > 0 && !staging_ok(grad, esize(grad_dtype), lp_out, n))
        return fail(ZERO_EINVAL, "%s: lp_out overlaps grad other than as the same 16-bit array", fn);
    int sk = 0;
    zf::offload_adam_host(grad, grad_dtype, master, exp_avg, exp_avg_sq, n, lp_out, param_dtype, *hp,
                          *host_state, n_threads, &sk);
    *skipped = sk;
    return ok();
}

int zero_offload_step(const void* d_grad, int32_t grad_dtype, int64_t n, float* h_master,
                      float* h_exp_avg, float* h_exp_avg_sq, void* h_grad_stage, void* h_lp_stage,
                      void* d_allgather, int32_t param_dtype, int64_t slot_offset,
                      const zero_adamw_hparams_t* hp, zero_step_state_t* d_state, int64_t chunk,
                      int32_t n_threads, void* stream) {
    const char* fn = "zero_offload_step";
    if (int e = check_hp(fn, hp)) return e;
    if (!d_state) return fail(ZERO_EINVAL, "%s: NULL state", fn);
    if (!aligned(d_state, 8)) return fail(ZERO_EALIGN, "%s: state not 8-byte aligned", fn);
    if (!valid_dtype(grad_dtype)) return fail(ZERO_EINVAL, "%s: bad grad_dtype %d", fn, grad_dtype);
    if (param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: param_dtype must be fp16 or bf16", fn);
    if (n < 0 || slot_offset < 0 || chunk < 0 || n_threads < 0)
        return fail(ZERO_EINVAL, "%s: negative size, offset, chunk or thread count", fn);
    if (n > 0 && (!d_grad || !h_master || !h_exp_avg || !h_exp_avg_sq || !h_grad_stage ||
                  !h_lp_stage || !d_allgather))
        return fail(ZERO_EINVAL, "%s: NULL pointer", fn);
    const int es = esize(grad_dtype);
    if (n > 0 && (!aligned(d_grad, es) || !aligned(h_grad_stage, es) || !aligned(h_master, 4) ||
                  !aligned(h_exp_avg, 4) || !aligned(h_exp_avg_sq, 4) || !aligned(h_lp_stage, 2) ||
                  !aligned(d_allgather, 2)))
        return fail(ZERO_EALIGN, "%s: a buffer is not aligned to its element size", fn);
    // chunks of one buffer are filled while other chunks of the other are
    // read: the two are disjoint, or one 16-bit buffer used in place
    if (n > 0 && !staging_ok(h_grad_stage, es, h_lp_stage, n))
        return fail(ZERO_EINVAL, "%s: the staging buffers overlap other than as one 16-bit buffer", fn);
    zf::OffloadLaunch a;
    memset(&a, 0, sizeof a);
    a.d_grad = d_grad;
    a.gdtype = grad_dtype;
    a.pdtype = param_dtype;
    a.n = n;
    a.h_p = h_master;
    a.h_m = h_exp_avg;
    a.h_v = h_exp_avg_sq;
    a.h_grad = h_grad_stage;
    a.h_lp = h_lp_stage;
    a.d_slot = n > 0 ? static_cast<uint16_t*>(d_allgather) + slot_offset : nullptr;
    a.chunk = chunk > 0 ? chunk : (int64_t)1 << 24;
    a.n_threads = n_threads;
    a.st = d_state;
    const int e = zf::offload_step(a, *hp, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}

// ---------------------------------------------------------------------------
// INT8 All-Gather consumer ("DeepSpeed 与 FSDP", ZeRO++：量化通信压缩;
// 2kiu.com §4.2): the gathered slots back to the flat parameter.
int zero_dequant_allgather(const int8_t* q_buf, const float* q_scales, int32_t n_slots,
                           int64_t slot_numel, int32_t block, void* out, int32_t out_dtype,
                           void* stream) {
    const char* fn = "zero_dequant_allgather";
    if (!valid_dtype(out_dtype)) return fail(ZERO_EINVAL, "%s: bad out_dtype %d", fn, out_dtype);
    if (n_slots < 1 || n_slots > 65536) return fail(ZERO_ERANGE, "%s: n_slots %d not in [1, 65536]", fn, n_slots);
    if (slot_numel < 0) return fail(ZERO_EINVAL, "%s: negative slot_numel", fn);
    if (block < 4 || block % 4 != 0) return fail(ZERO_EINVAL, "%s: block %d is not a positive multiple of 4", fn, block);
    int64_t total = 0;
    if (!mul_ok(slot_numel, n_slots, &total) || !mul_ok(total, 4, &total))
        return fail(ZERO_ERANGE, "%s: n_slots * slot_numel overflows", fn);
    if (slot_numel == 0) return ok();
    if (!q_buf || !q_scales || !out) return fail(ZERO_EINVAL, "%s: NULL pointer", fn);
    const int es = esize(out_dtype);
    if (!aligned(q_scales, 4) || !aligned(out, es)) return fail(ZERO_EALIGN, "%s: misaligned", fn);
    zf::DequantLaunch a;
    memset(&a, 0, sizeof a);
    a.q = q_buf;
    a.qs = q_scales;
    a.out = out;
    a.out_dtype = out_dtype;
    a.block = block;
    a.n_slots = n_slots;
    a.slot_numel = slot_numel;
    // quad path: 4 codes (4 B) in, 4 outputs (8 B 16-bit, 16 B fp32) out per
    // lane; slot starts keep the alignment when slot_numel % 4 == 0
    a.vec = (slot_numel % 4 == 0 && aligned(q_buf, 4) && aligned(out, 4 * es)) ? 1 : 0;
    const int e = zf::launch_dequant(a, stream);
    if (e) return hip_fail(e, fn);
    return ok();
}

}  // extern "C"
