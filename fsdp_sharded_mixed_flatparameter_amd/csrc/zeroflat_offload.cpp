// zeroflat_offload.cpp -- ZeRO-Offload: the rank's AdamW step on host cores.
//
// "DeepSpeed 与 FSDP", ZeRO-Offload: the fp32 optimizer state (master, m, v)
// lives in CPU memory and the Adam update runs on the CPU; the 16-bit
// gradients travel to the host and the updated 16-bit parameters back.
// 2kiu.com §4.1 (states moved to CPU memory) and §5.1 (offload_optimizer on
// cpu with pinned memory).
//
// The host update is the same binary32 sequence as the GPU kernel (the step's
// definition in zeroflat.h): every operation rounded once, no FMA (built with
// -ffp-contract=off), IEEE division and square root (the SIMD instructions are
// correctly rounded), 16-bit rounding on the bit patterns.  So a step computed
// here equals the GPU's bit for bit.  The inner loop is built for AVX-512,
// AVX2 and baseline x86-64 and picked at load time (target_clones); threads
// split each chunk into contiguous parts.
//
// zero_offload_step pipelines the transfers around it: the gradient shard
// moves device-to-host in chunks on the caller's stream, each chunk is updated
// as soon as its copy has landed, and its 16-bit parameters move host-to-device
// into the All-Gather slot while later chunks are still being computed.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "zeroflat.h"
#include "zf_launch.h"

namespace zf {
namespace {

// ---------------------------------------------------------------- formats (host)
inline uint32_t fbits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return u;
}
inline float bitsf(uint32_t u) {
    float x;
    memcpy(&x, &u, 4);
    return x;
}
// binary16 -> binary32 (exact), branch-free so that it vectorizes
inline float h2f(uint32_t h) {
    const uint32_t sign = (h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu;
    const uint32_t mnt = h & 0x3ffu;
    const uint32_t normal = ((e + 112u) << 23) | (mnt << 13);
    const uint32_t special = 0x7f800000u | (mnt << 13);
    const float sub = (float)(int32_t)mnt * 0x1p-24f;  // exact: < 2^10 * 2^-24
    uint32_t r = e == 31u ? special : normal;
    r = e == 0u ? fbits(sub) : r;
    return bitsf(sign | r);
}
inline float b2f(uint32_t h) { return bitsf(h << 16); }
// binary32 -> binary16 / bfloat16, round to nearest, ties to even, on the bits;
// NaN -> the canonical quiet NaN with the sign kept
inline uint32_t f2h(float x) {
    const uint32_t u = fbits(x);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7fffffffu;
    const uint32_t m = a - 0x38000000u;                           // exponent bias 127 -> 15
    const uint32_t hn = (m + 0xfffu + ((m >> 13) & 1u)) >> 13;    // normal: round at bit 13
    const uint32_t hs = fbits(bitsf(a) + 0.5f) - 0x3f000000u;     // subnormal: quantum 2^-24
    uint32_t h = a >= 0x38800000u ? hn : hs;
    h = a >= 0x477ff000u ? 0x7c00u : h;                           // >= 65520 -> infinity
    h = a > 0x7f800000u ? 0x7e00u : h;                            // NaN
    return sign | h;
}
inline uint32_t f2b(float x) {
    const uint32_t u = fbits(x);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7fffffffu) > 0x7f800000u ? (((u >> 16) & 0x8000u) | 0x7fc0u) : r;
}

struct Scalars {
    float inv, coef, b1, c1, b2, c2, bc1, bc2, lr, wdf, eps;
};

template <int GT>
inline float grad_at(const void* g, int64_t i) {
    if constexpr (GT == ZERO_F32) return static_cast<const float*>(g)[i];
    else if constexpr (GT == ZERO_F16) return h2f(static_cast<const uint16_t*>(g)[i]);
    else return b2f(static_cast<const uint16_t*>(g)[i]);
}

// g and lp may be the same 16-bit array (in-place staging: the chunk's
// gradients are overwritten by its parameters).  Each block of kHostBlock
// elements first reads its gradients into a local array and only then
// computes and stores, so every element's gradient is read before its slot is
// written, and both loops still vectorize (p, m and v are restrict; the local
// array cannot alias lp).
constexpr int kHostBlock = 64;

template <int GT, int PT>
__attribute__((always_inline)) inline void adam_loop(const Scalars& s, const void* g,
                                                     float* __restrict__ p, float* __restrict__ m,
                                                     float* __restrict__ v, uint16_t* lp,
                                                     int64_t lo, int64_t hi) {
    for (int64_t i0 = lo; i0 < hi; i0 += kHostBlock) {
        const int nb = hi - i0 < kHostBlock ? (int)(hi - i0) : kHostBlock;
        float gb[kHostBlock];
        for (int j = 0; j < nb; ++j) gb[j] = grad_at<GT>(g, i0 + j);
        for (int j = 0; j < nb; ++j) {
            const int64_t i = i0 + j;
            const float u = gb[j] * s.inv;               // unscale
            const float gg = u * s.coef;                 // clip
            const float mn = s.b1 * m[i] + s.c1 * gg;
            const float vn = s.b2 * v[i] + s.c2 * (gg * gg);
            const float mh = mn / s.bc1;
            const float vh = vn / s.bc2;
            const float d = __builtin_sqrtf(vh) + s.eps;
            const float pn = p[i] * s.wdf - (s.lr * mh) / d;
            p[i] = pn;
            m[i] = mn;
            v[i] = vn;
            lp[i] = (uint16_t)(PT == ZERO_F16 ? f2h(pn) : f2b(pn));
        }
    }
}

// One contiguous range of the update; one machine-code clone per ISA level.
__attribute__((target_clones("avx512f", "avx2", "default"))) void adam_range(
    const Scalars& s, int gdt, int pdt, const void* g, float* p, float* m, float* v,
    uint16_t* lp, int64_t lo, int64_t hi) {
#define ZF_OFF(GT, PT) \
    if (gdt == GT && pdt == PT) return adam_loop<GT, PT>(s, g, p, m, v, lp, lo, hi);
    ZF_OFF(ZERO_F32, ZERO_F16) ZF_OFF(ZERO_F32, ZERO_BF16)
    ZF_OFF(ZERO_F16, ZERO_F16) ZF_OFF(ZERO_F16, ZERO_BF16)
    ZF_OFF(ZERO_BF16, ZERO_F16) ZF_OFF(ZERO_BF16, ZERO_BF16)
#undef ZF_OFF
}

// The same per-step decisions as the device prologue, from a host copy of
// the state: skip on any overflow; clip coefficient in binary64 rounded once;
// exact reciprocal of the power-of-two loss scale; bias corrections at
// t = step + 1 from the stored beta powers.
bool step_scalars(const zero_step_state_t& st, const zero_adamw_hparams_t& hp, Scalars* s) {
    if ((st.overflow | st.remote_overflow) != 0) return false;
    const double total = st.sumsq + st.remote_sumsq;
    s->coef = 1.0f;
    if (hp.max_grad_norm > 0.0) {
        const double c = hp.max_grad_norm / (sqrt(total) + 1e-6);
        s->coef = (float)(c < 1.0 ? c : 1.0);
    }
    s->inv = (float)(1.0 / (double)st.loss_scale);
    s->bc1 = (float)(1.0 - st.beta1_pow * hp.beta1);
    s->bc2 = (float)(1.0 - st.beta2_pow * hp.beta2);
    s->b1 = (float)hp.beta1;
    s->c1 = (float)(1.0 - hp.beta1);
    s->b2 = (float)hp.beta2;
    s->c2 = (float)(1.0 - hp.beta2);
    s->lr = (float)hp.lr;
    s->wdf = (float)(1.0 - hp.lr * hp.weight_decay);
    s->eps = (float)hp.eps;
    return true;
}

// Fixed-size worker pool for one call: run(lo, hi) splits [lo, hi) into
// n contiguous parts (multiples of 64 elements) and returns when all are done.
class Pool {
   public:
    explicit Pool(int n) : n_(n) {
        for (int t = 1; t < n_; ++t) threads_.emplace_back([this, t] { worker(t); });
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> l(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& th : threads_) th.join();
    }
    void run(int64_t lo, int64_t hi, const std::function<void(int64_t, int64_t)>& fn) {
        {
            std::lock_guard<std::mutex> l(mu_);
            lo_ = lo;
            hi_ = hi;
            fn_ = &fn;
            pending_ = n_ - 1;
            ++gen_;
        }
        cv_.notify_all();
        part(0);
        std::unique_lock<std::mutex> l(mu_);
        done_.wait(l, [this] { return pending_ == 0; });
    }

   private:
    void part(int t) {
        const int64_t n = hi_ - lo_;
        int64_t per = (n + n_ - 1) / n_;
        per = (per + 63) / 64 * 64;
        const int64_t a = std::min(hi_, lo_ + per * t);
        const int64_t b = std::min(hi_, a + per);
        if (a < b) (*fn_)(a, b);
    }
    void worker(int t) {
        uint64_t seen = 0;
        for (;;) {
            {
                std::unique_lock<std::mutex> l(mu_);
                cv_.wait(l, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
            }
            part(t);
            {
                std::lock_guard<std::mutex> l(mu_);
                if (--pending_ == 0) done_.notify_one();
            }
        }
    }
    int n_;
    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable cv_, done_;
    bool stop_ = false;
    uint64_t gen_ = 0;
    int pending_ = 0;
    int64_t lo_ = 0, hi_ = 0;
    const std::function<void(int64_t, int64_t)>* fn_ = nullptr;
};

int threads_for(int32_t n_threads) {
    if (n_threads > 0) return n_threads;
    const unsigned hc = std::thread::hardware_concurrency();
    return hc > 0 ? (int)hc : 1;
}

}  // namespace

int offload_adam_host(const void* g, int32_t gdt, float* p, float* m, float* v, int64_t n,
                      void* lp, int32_t pdt, const zero_adamw_hparams_t& hp,
                      const zero_step_state_t& st, int32_t n_threads, int* skipped) {
    Scalars s;
    *skipped = step_scalars(st, hp, &s) ? 0 : 1;
    if (*skipped || n == 0) return 0;
    Pool pool(std::min<int64_t>(threads_for(n_threads), std::max<int64_t>(1, n / 4096)));
    const std::function<void(int64_t, int64_t)> fn = [&](int64_t a, int64_t b) {
        adam_range(s, gdt, pdt, g, p, m, v, static_cast<uint16_t*>(lp), a, b);
    };
    pool.run(0, n, fn);
    return 0;
}

int offload_step(const OffloadLaunch& a, const zero_adamw_hparams_t& hp, void* stream_v) {
    hipStream_t stream = (hipStream_t)stream_v;
    const int64_t es = a.gdtype == ZERO_F32 ? 4 : 2;
    const int64_t nch = a.n == 0 ? 0 : (a.n + a.chunk - 1) / a.chunk;
    // the scalars of the state (everything before the per-block partials)
    std::unique_ptr<zero_step_state_t> host_st(new zero_step_state_t);
    zero_step_state_t& st = *host_st;
    hipEvent_t ev_state = nullptr;
    hipError_t e = hipMemcpyAsync(&st, a.st, offsetof(zero_step_state_t, partials),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_state, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev_state, stream);
    std::vector<hipEvent_t> ev(nch, nullptr);
    for (int64_t c = 0; c < nch && e == hipSuccess; ++c) {
        const int64_t lo = c * a.chunk, len = std::min(a.chunk, a.n - lo);
        e = hipMemcpyAsync(static_cast<char*>(a.h_grad) + lo * es,
                           static_cast<const char*>(a.d_grad) + lo * es, len * es,
                           hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev[c], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(ev[c], stream);
    }
    if (e == hipSuccess) e = hipEventSynchronize(ev_state);  // the state only
    Scalars s;
    const int skipped = e == hipSuccess && !step_scalars(st, hp, &s);
    // parameters go up on a stream of their own (default priority), so that the
    // link carries both directions at once
    hipStream_t up = nullptr;
    if (e == hipSuccess && !skipped && a.n > 0) e = hipStreamCreateWithFlags(&up, hipStreamNonBlocking);
    if (e == hipSuccess && !skipped && a.n > 0) {
        // Every thread walks all chunks in order and updates its own part of
        // each (the same split as the host entry point) as soon as the chunk's
        // gradient has landed; the thread that finishes a chunk last sends its
        // parameters up.  No barrier between chunks, so a thread that is
        // ahead goes on with the next chunk instead of waiting for the slowest.
        const int nt = (int)std::min<int64_t>(threads_for(a.n_threads),
                                              std::max<int64_t>(1, a.chunk / 4096));
        uint16_t* lp = static_cast<uint16_t*>(a.h_lp);
        std::vector<std::atomic<int>> left(nch);
        for (auto& x : left) x.store(nt);
        std::atomic<int> err(hipSuccess);
        auto worker = [&](int t) {
            for (int64_t c = 0; c < nch; ++c) {
                if (err.load(std::memory_order_relaxed) != hipSuccess) return;
                const int64_t lo = c * a.chunk, len = std::min(a.chunk, a.n - lo);
                hipError_t we = hipEventSynchronize(ev[c]);
                if (we == hipSuccess) {
                    int64_t per = (len + nt - 1) / nt;
                    per = (per + 63) / 64 * 64;
                    const int64_t pa = std::min(lo + len, lo + per * t);
                    const int64_t pb = std::min(lo + len, pa + per);
                    if (pa < pb)
                        adam_range(s, a.gdtype, a.pdtype, a.h_grad, a.h_p, a.h_m, a.h_v, lp, pa, pb);
                    if (left[c].fetch_sub(1) == 1)
                        we = hipMemcpyAsync(static_cast<uint16_t*>(a.d_slot) + lo, lp + lo, len * 2,
                                            hipMemcpyHostToDevice, up);
                }
                if (we != hipSuccess) {
                    int none = hipSuccess;
                    err.compare_exchange_strong(none, (int)we);
                    return;
                }
            }
        };
        std::vector<std::thread> pool;
        for (int t = 1; t < nt; ++t) pool.emplace_back(worker, t);
        worker(0);
        for (auto& th : pool) th.join();
        e = (hipError_t)err.load();
    }
    if (up) {
        const hipError_t e2 = hipStreamSynchronize(up);
        if (e == hipSuccess) e = e2;
        (void)hipStreamDestroy(up);
    }
    if (e != hipSuccess) (void)hipStreamSynchronize(stream);  // no copy may outlive the call
    for (auto x : ev)
        if (x) (void)hipEventDestroy(x);
    if (ev_state) (void)hipEventDestroy(ev_state);
    if (e != hipSuccess) return (int)e;
    // loss scaler, counters and accumulators on the device, as after a GPU step
    AdamLaunch f;
    memset(&f, 0, sizeof f);
    f.n = 0;
    f.flags = ZERO_STEP_FINALIZE;
    f.beta1 = hp.beta1;
    f.beta2 = hp.beta2;
    f.max_norm = hp.max_grad_norm;
    f.st = a.st;
    const int fe = launch_adamw(f, stream);
    if (fe) return fe;
    return (int)hipStreamSynchronize(stream);  // the host buffers are free again
}

}  // namespace zf
