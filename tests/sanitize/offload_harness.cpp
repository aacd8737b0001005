// CPU harness for the ZeRO-Offload host code (zeroflat_offload.cpp) under a
// sanitizer (ThreadSanitizer, or AddressSanitizer + UndefinedBehaviorSanitizer).
//
// The eight HIP runtime calls of zf::offload_step are emulated on the host:
// copies are synchronous memcpy, events and streams complete at once, and the
// device finalize is a no-op.  So the threaded chunk walk, the per-chunk
// last-arriver counters and the uploads issued from worker threads run as in
// the library, over host arrays standing in for device memory.
//
// For each size, chunk, thread count and staging mode (two buffers, or one
// 16-bit buffer used in place) the pipelined step and the thread-pool host
// step must equal a one-thread host step bit for bit, and the slot's
// neighbours must stay untouched.  Prints "ok" and exits 0 on success.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <vector>

#include "zf_launch.h"

static char g_handles[64];
extern "C" {
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = reinterpret_cast<hipEvent_t>(g_handles);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
    *s = reinterpret_cast<hipStream_t>(g_handles + 8);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
}
namespace zf {
int launch_adamw(const AdamLaunch&, void*) { return 0; }  // the device finalize
}

static uint32_t next(uint64_t& s) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
}

int main() {
    const zero_adamw_hparams_t hp = {3e-5, 0.9, 0.999, 1e-8, 0.01, 1.0};
    zero_step_state_t* st = new zero_step_state_t;
    memset(st, 0, sizeof *st);
    st->loss_scale = 1024.0f;
    st->min_scale = 1.0f;
    st->step = 1;
    st->beta1_pow = 0.9;
    st->beta2_pow = 0.999;
    st->sumsq = 2.0;   // clipped: norm sqrt(2) > 1
    int bad = 0, cases = 0;
    for (int64_t n : {1, 5000, 100003}) {
        uint64_t s = 11 + (uint64_t)n;
        std::vector<uint16_t> dg(n);  // fp16 gradient, stands in for device memory
        for (auto& x : dg) x = (uint16_t)((0x1400 + (next(s) & 0x3ff)) | ((next(s) & 1) << 15));
        std::vector<float> p0(n);
        for (auto& x : p0) x = (float)((int)(next(s) % 2001) - 1000) * 1e-5f;
        std::vector<float> rp = p0, rm(n, 0.f), rv(n, 0.f);
        std::vector<uint16_t> rlp(n);
        int sk = -1;
        if (zf::offload_adam_host(dg.data(), ZERO_F16, rp.data(), rm.data(), rv.data(), n,
                                  rlp.data(), ZERO_F16, hp, *st, 1, &sk) != 0 || sk != 0) {
            printf("reference step failed\n");
            return 1;
        }
        for (int64_t chunk : {4096, 10000, 65536}) {
            for (int threads : {2, 5, 8}) {
                for (int inplace = 0; inplace < 2; ++inplace) {
                    ++cases;
                    // the pipelined step
                    std::vector<float> p = p0, m(n, 0.f), v(n, 0.f);
                    std::vector<uint16_t> gstage(n), lpstage(n), slot(n + 8, 0);
                    zf::OffloadLaunch a;
                    memset(&a, 0, sizeof a);
                    a.d_grad = dg.data();
                    a.gdtype = ZERO_F16;
                    a.pdtype = ZERO_F16;
                    a.n = n;
                    a.h_p = p.data();
                    a.h_m = m.data();
                    a.h_v = v.data();
                    a.h_grad = gstage.data();
                    a.h_lp = inplace ? gstage.data() : lpstage.data();
                    a.d_slot = slot.data() + 4;
                    a.chunk = chunk;
                    a.n_threads = threads;
                    a.st = st;
                    const int rc = zf::offload_step(a, hp, nullptr);
                    const bool edges = slot[0] | slot[1] | slot[2] | slot[3] | slot[n + 4] | slot[n + 7];
                    if (rc != 0 || memcmp(rp.data(), p.data(), n * 4) || memcmp(rm.data(), m.data(), n * 4) ||
                        memcmp(rv.data(), v.data(), n * 4) || memcmp(rlp.data(), slot.data() + 4, n * 2) || edges) {
                        printf("offload_step differs: n=%lld chunk=%lld threads=%d in_place=%d rc=%d\n",
                               (long long)n, (long long)chunk, threads, inplace, rc);
                        ++bad;
                    }
                    // the thread-pool host step over the same inputs
                    std::vector<float> q = p0, qm(n, 0.f), qv(n, 0.f);
                    std::vector<uint16_t> qg = dg, qlp(n);
                    int qsk = -1;
                    const int qrc = zf::offload_adam_host(qg.data(), ZERO_F16, q.data(), qm.data(), qv.data(), n,
                                                          inplace ? (void*)qg.data() : (void*)qlp.data(),
                                                          ZERO_F16, hp, *st, threads, &qsk);
                    const uint16_t* qout = inplace ? qg.data() : qlp.data();
                    if (qrc != 0 || qsk != 0 || memcmp(rp.data(), q.data(), n * 4) ||
                        memcmp(rlp.data(), qout, n * 2)) {
                        printf("offload_adam_host differs: n=%lld threads=%d in_place=%d\n", (long long)n,
                               threads, inplace);
                        ++bad;
                    }
                }
            }
        }
    }
    delete st;
    if (bad) {
        printf("FAILED %d of %d\n", bad, cases);
        return 1;
    }
    printf("ok %d cases\n", cases);
    return 0;
}
