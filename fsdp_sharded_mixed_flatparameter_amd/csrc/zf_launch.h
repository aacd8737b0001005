// zf_launch.h -- internal interface between the C-ABI layer (zeroflat_api.cpp)
// and the gfx950 kernels (zeroflat_kernels.hip).  Arguments reaching these
// launchers have been validated; they only pick a kernel variant and launch.
#pragma once

#include <stdint.h>

#include "zeroflat.h"

namespace zf {

// Reduce (n_ranks buffers) or statistics-only (n_ranks == 1, red_out == null)
// over [0, n) of each buffer (pointers already offset to the rank's slice).
struct ReduceLaunch {
    const void* bufs[ZERO_MAX_RANKS];
    int32_t n_ranks;
    int32_t dtype;   // zero_dtype_t of the inputs
    int32_t op;      // zero_reduce_op_t
    int32_t vec;     // 1: vector path (every pointer allows quad accesses, from
                     // element `head` on for the inputs)
    int32_t head;    // vector path: elements 0 .. head-1 precede the inputs' first
                     // 128-byte line boundary (0..63; the output is 16-byte
                     // aligned at element 0)
    int64_t n;
    float* red_out;  // may be null
    int32_t accumulate;     // 1: red_out += reduce (red_out is read, then written)
    int32_t block;          // INT8 payload only: elements per scale
    int32_t block_shift;    // log2(block) if a power of two, else -1
    zero_step_state_t* st;  // may be null
    double* partials;       // per-block partial sums of the statistics (st set):
                            // st->partials, or the library's scratch
};
int launch_reduce_stats(const ReduceLaunch& a, void* stream);
// The same launch with the statistics' partial sums in the library's own
// device scratch (one array per device, found on the first call on a device)
// instead of the state's table; the state then needs only its header.
int launch_reduce_noalloc(ReduceLaunch& a, void* stream);
// The quantised-gradient reduce: bufs[2k] = rank k's INT8 codes, bufs[2k+1]
// its fp32 block scales (n_ranks <= ZERO_MAX_RANKS / 2).
int launch_reduce_q8(const ReduceLaunch& a, void* stream);

struct AdamLaunch {
    const void* g;
    int32_t gdtype;
    int32_t pdtype;
    float* p;
    float* m;
    float* v;
    int64_t n;
    void* lp;        // All-Gather slot, already offset
    int8_t* q;       // INT8 slot, already offset (or null)
    float* qs;       // scales of the slot, already offset
    int32_t vec;     // 1: vector path allowed
    uint32_t flags;
    float b1, c1, b2, c2, lr, wdf, eps;
    double beta1, beta2, max_norm;
    zero_step_state_t* st;
};
int launch_adamw(const AdamLaunch& a, void* stream);

struct QuantLaunch {
    const void* x;
    int32_t dtype;
    int32_t vec;     // 2: eight elements per lane (x 16-byte, q 8-byte aligned);
                     // 1: quad tiles (x 8-byte, q 4-byte aligned); 0: element-wise
    int64_t n;
    int8_t* q;
    float* qs;
};
int launch_quant(const QuantLaunch& a, void* stream);

// Dequantise n_slots INT8 slots of slot_numel codes into the flat buffer.
struct DequantLaunch {
    const int8_t* q;
    const float* qs;
    void* out;
    int32_t out_dtype;
    int32_t block;
    int32_t n_slots;
    int32_t vec;     // 1: slot_numel % 4 == 0 and every pointer allows quad accesses
    int64_t slot_numel;
};
int launch_dequant(const DequantLaunch& a, void* stream);

// ZeRO-Offload (zeroflat_offload.cpp).  The host update over host arrays:
// *skipped = 1 (and nothing written) when the state says overflow.
int offload_adam_host(const void* g, int32_t gdt, float* p, float* m, float* v, int64_t n,
                      void* lp, int32_t pdt, const zero_adamw_hparams_t& hp,
                      const zero_step_state_t& st, int32_t n_threads, int* skipped);
// The pipelined step: gradient chunks device->host, host update, 16-bit
// parameter chunks host->device into the slot, then the device finalize.
// Blocks the calling thread until every copy has completed.
struct OffloadLaunch {
    const void* d_grad;
    int32_t gdtype;
    int32_t pdtype;
    int64_t n;
    float* h_p;
    float* h_m;
    float* h_v;
    void* h_grad;     // pinned staging, n gradient elements
    void* h_lp;       // pinned staging, n 16-bit parameters
    void* d_slot;     // the All-Gather slot, already offset
    int64_t chunk;
    int32_t n_threads;
    zero_step_state_t* st;
};
int offload_step(const OffloadLaunch& a, const zero_adamw_hparams_t& hp, void* stream);

const char* hip_error_string(int err);

}  // namespace zf
