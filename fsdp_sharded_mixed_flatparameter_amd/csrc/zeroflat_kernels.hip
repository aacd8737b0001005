// zeroflat_kernels.hip -- gfx950 (MI355X, CDNA4, wave64) kernels of one
// rank's sharded mixed-precision AdamW step over a FlatParameter:
//   reduce_kernel    N-way reduce of the rank buffers (fp32/fp16/bf16, or INT8
//                    codes with block scales), optionally added into the fp32
//                    shard (gradient accumulation), fused with the step
//                    statistics; with one buffer and no output, the statistics
//                    pass of a pre-reduced shard
//   fold_kernel      the statistics' per-block partial sums, in a fixed order
//   adamw_kernel     skip/clip prologue, fused AdamW, 16-bit write-back, INT8
//   adamw_sched_kernel  the same for large shards: a persistent grid taking
//                    groups of tiles from a counter in the state
//   finalize_kernel  loss scaler and counters
//   quant_kernel     INT8 of an existing 16-bit slot (quad tiles)
//   quant8_kernel    the same on 16-byte aligned slots, eight elements per lane
//   dequant_kernel   the INT8 All-Gather consumer, tiles per slot
//   dequant_flat_kernel  the same with tiles over the flat output (slots of
//                    2048 elements or more)
//
// Every kernel here streams HBM once: none is a contraction, so there is no
// MFMA work; the design goals are wide coalesced accesses, enough bytes in
// flight per CU, and the per-element fp32 operation order fixed by the step's
// definition (zeroflat.h), so results equal a plain IEEE evaluation bit for
// bit.  Built with -ffp-contract=off (no FMA fusion) and correctly rounded
// fp32 division and square root.
//
// Data mapping ("quad" tiles): a wavefront owns tiles of 256*kU consecutive
// elements; in slice u of a tile, lane l holds elements 256u + 4l .. 4l+3, so
// each fp32 array moves as one 16-byte access per lane (1 KiB per wave
// instruction) and each 16-bit array as one 8-byte access.  One slice of 256
// elements is exactly one INT8 block, reduced across the wave.  All kU
// slices' loads are issued before any arithmetic (bytes in flight per lane),
// and every stream uses non-temporal loads/stores: each byte is touched once.
// The AdamW grid holds one tile per wave, issued in launch slices over tile
// ranges; a large shard takes its tiles from a counter instead
// (adamw_sched_kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "zf_launch.h"

namespace zf {
namespace {

// Launch shape.  ZF_ADAM_U (256-element slices per wave tile) trades bytes in
// flight per lane against occupancy; ZF_ADAM_GRID caps the AdamW/quant grid
// (0: one tile per wave, blocks dispatched as earlier ones retire).
#ifndef ZF_ADAM_U
#define ZF_ADAM_U 4
#endif
#ifndef ZF_ADAM_GRID
#define ZF_ADAM_GRID 0
#endif
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kU = ZF_ADAM_U;               // 256-element slices per adamw/quant tile
constexpr int64_t kTile = 256 * kU;         // adamw/quant tile (elements per wave)
// Streaming kernels loop over tiles when the grid is capped; 2^22 blocks of
// 256 threads keep every launch inside HIP's 2^32-thread grid limit.
constexpr int kMaxGridStream = 1 << 22;
constexpr int kMaxGridStep = ZF_ADAM_GRID > 0 ? ZF_ADAM_GRID : kMaxGridStream;
constexpr int kMaxGridReduce = ZERO_MAX_PARTIALS;

// Launch slices and an occupancy cap for the long streaming kernels.  One
// launch of a few hundred thousand blocks streams a little slower than the
// same tiles issued as consecutive launches of kSliceBlocks blocks (tile
// ranges [t0, t1), same stream): on the 1.25e9-element update 6.24-6.38 ms
// as one launch against 5.86-5.96 ms in slices of 16,384 or 32,768 blocks,
// and the 8-slice reduce and the INT8 gather gained 3-6% the same way.  A kernel
// boundary makes every XCD finish before the next range starts, which keeps
// the addresses in flight in one window; within one long launch the
// dispatch order alone does not.  kLdsTwoBlocks is a dynamic LDS reservation
// (unused by the kernel) that lets only two 256-thread blocks reside per
// compute unit (160 KiB of LDS): the update and the wide reduces, whose
// waves each keep 16-32 KiB of reads in flight, ran another 1-5% faster so;
// kernels with fewer bytes in flight per wave (the statistics pass, the
// INT8 quantiser and gather) ran 30-70% slower and keep full occupancy, and
// so do launches of fewer than kTwoBlocksMin blocks (the 7B block's reduce,
// 6,200 blocks, ran 1-2% slower with the cap) and the update with the INT8
// epilogue when issued in slices (on the 70B shard 5.85 against 5.35 ms
// without the cap; a shard that large now takes the counter-scheduled form).
constexpr int64_t kSliceBlocks = 32768;
constexpr unsigned kLdsTwoBlocks = 56 * 1024;
constexpr int64_t kTwoBlocksMin = 8192;
// the counter-scheduled update (adamw_sched_kernel) from this many tile groups
constexpr int64_t kSchedMinGroups = 8192;

// Native vectors for the non-temporal (streaming, read-once / write-once)
// accesses: every array of the step is touched exactly once per launch.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f ldnt_f4(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ void stnt_f4(float* p, float a, float b, float c, float d) {
    v4f x;
    x.x = a; x.y = b; x.z = c; x.w = d;
    __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(p));
}
__device__ __forceinline__ v2u ldnt_u2(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
}
__device__ __forceinline__ void stnt_u2(void* p, uint32_t a, uint32_t b) {
    v2u x;
    x.x = a; x.y = b;
    __builtin_nontemporal_store(x, reinterpret_cast<v2u*>(p));
}
__device__ __forceinline__ void stnt_u1(void* p, uint32_t a) {
    __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
}

// Buffer (descriptor) accesses for the update's full tiles: a raw-buffer
// resource over one wave's tile of one array, whose base is wave-uniform and
// so lives in scalar registers; each lane supplies only a 32-bit byte offset.
// The cache-policy operand is non-temporal, as for the global accesses: on
// the update's arrays, plain stores and the sc0 / sc1 encodings (with or
// without nt) measured 1-4% slower.  The update runs at the rate of the same
// accesses as global instructions (within 0.2% on the same arrays); the
// resource also bounds every access to its tile in hardware: an access past
// the resource's size is dropped, and full tiles make none.
constexpr int kBufWord3 = 0x00020000;   // gfx9-family raw-buffer descriptor, word 3
constexpr int kPolicyNT = 2;            // cache-policy operand: non-temporal
typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes buf_res(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                             kBufWord3);
}
__device__ __forceinline__ v4u bld_u4(BufRes r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyNT);
}
__device__ __forceinline__ v2u bld_u2(BufRes r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyNT);
}
__device__ __forceinline__ void bst_u4(BufRes r, uint32_t off, v4u x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)off, 0, kPolicyNT);
}
__device__ __forceinline__ void bst_u2(BufRes r, uint32_t off, v2u x) {
    __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)off, 0, kPolicyNT);
}
__device__ __forceinline__ void bst_u1(BufRes r, uint32_t off, uint32_t x) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, (int)off, 0, kPolicyNT);
}

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float b2f(uint32_t h) { return __uint_as_float(h << 16); }
// binary32 -> binary16 / bfloat16 rounding to nearest, ties to even, written
// on the bit patterns so that no hardware conversion mode is involved.
__device__ __forceinline__ uint32_t f2h(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t h;
    if (a >= 0x7f800000u) {
        h = a > 0x7f800000u ? 0x7e00u : 0x7c00u;           // quiet NaN / infinity
    } else if (a >= 0x477ff000u) {
        h = 0x7c00u;                                        // >= 65520 rounds to infinity
    } else if (a >= 0x38800000u) {                          // normal binary16 (>= 2^-14)
        const uint32_t m = a - 0x38000000u;                 // exponent bias 127 -> 15
        h = (m + 0xfffu + ((m >> 13) & 1u)) >> 13;          // round at bit 13, ties to even
    } else {                                                // subnormal binary16: quantum 2^-24,
        h = __float_as_uint(__uint_as_float(a) + 0.5f) - 0x3f000000u;  // the ulp of 0.5
    }
    return sign | h;
}
__device__ __forceinline__ uint32_t f2b(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;          // round at bit 16, ties to even
}

template <int DT>
__device__ __forceinline__ float cvt16(uint32_t h) {
    return DT == ZERO_F16 ? h2f(h) : b2f(h);
}
template <int DT>
__device__ __forceinline__ uint32_t round16(float x) {
    return DT == ZERO_F16 ? f2h(x) : f2b(x);
}

template <int DT>
__device__ __forceinline__ float load_one(const void* p, int64_t i) {
    if constexpr (DT == ZERO_F32) return static_cast<const float*>(p)[i];
    else return cvt16<DT>(static_cast<const uint16_t*>(p)[i]);
}

// four consecutive elements at byte offset off of a buffer resource (16-byte
// aligned for fp32, 8-byte for 16-bit formats)
template <int DT>
__device__ __forceinline__ void bload_quad(BufRes r, uint32_t off, float out[4]) {
    if constexpr (DT == ZERO_F32) {
        const v4u w = bld_u4(r, off);
        out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
        out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
    } else {
        const v2u w = bld_u2(r, off);
        out[0] = cvt16<DT>(w.x & 0xffffu);
        out[1] = cvt16<DT>(w.x >> 16);
        out[2] = cvt16<DT>(w.y & 0xffffu);
        out[3] = cvt16<DT>(w.y >> 16);
    }
}
__device__ __forceinline__ void bstore_f4(BufRes r, uint32_t off, const float x[4]) {
    v4u w;
    w.x = __float_as_uint(x[0]); w.y = __float_as_uint(x[1]);
    w.z = __float_as_uint(x[2]); w.w = __float_as_uint(x[3]);
    bst_u4(r, off, w);
}

// four consecutive elements from a 16-byte (fp32) or 8-byte (16-bit) aligned address
template <int DT>
__device__ __forceinline__ void load_quad(const void* p, int64_t i, float out[4]) {
    if constexpr (DT == ZERO_F32) {
        const v4f f = ldnt_f4(static_cast<const float*>(p) + i);
        out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
    } else {
        const v2u w = ldnt_u2(static_cast<const uint16_t*>(p) + i);
        out[0] = cvt16<DT>(w.x & 0xffffu);
        out[1] = cvt16<DT>(w.x >> 16);
        out[2] = cvt16<DT>(w.y & 0xffffu);
        out[3] = cvt16<DT>(w.y >> 16);
    }
}

// This wave's index in the grid, made a scalar (wave-uniform) value: loop
// bounds and tile indices derived from it then live in SGPRs, so per-tile
// pointers (the rank-buffer table in the kernel arguments) are fetched with
// scalar loads, which do not wait in the vector-memory counter behind the
// streaming loads in flight.
__device__ __forceinline__ int64_t wave_index() {
    return (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ double wave_sum(double x) {
    // xor butterfly: every lane ends with the same, order-fixed sum
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}
// block-wide sum, fixed order; the result is valid in thread 0
__device__ __forceinline__ double block_sum(double x) {
    __shared__ double sh[kWaves];
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += sh[w];
    }
    return t;
}

// ---------------------------------------------------------------- step scalars
struct StepScalars {
    int skip;
    float coef, inv, bc1, bc2;
};

// The per-step decisions, read from the device state by every block (and by
// the finalize kernel): overflow across ranks -> skip; global-norm clip
// coefficient; exact reciprocal of the power-of-two loss scale; bias
// corrections with t = step + 1.
__device__ __forceinline__ StepScalars read_step(const zero_step_state_t* st, double beta1,
                                                 double beta2, double max_norm) {
    StepScalars s;
    s.skip = (st->overflow | st->remote_overflow) != 0;
    const double total = st->sumsq + st->remote_sumsq;
    s.coef = 1.0f;
    if (max_norm > 0.0) {
        const double c = max_norm / (sqrt(total) + 1e-6);
        s.coef = (float)(c < 1.0 ? c : 1.0);
    }
    s.inv = (float)(1.0 / (double)st->loss_scale);
    s.bc1 = (float)(1.0 - st->beta1_pow * beta1);
    s.bc2 = (float)(1.0 - st->beta2_pow * beta2);
    return s;
}

// ---------------------------------------------------------------- reduce + statistics
// red[i] = sum over buffers in rank order (fp32), AVG -> / n_ranks; optional
// statistics of u = red * (1/loss_scale): per-block fp64 partial of u^2 into
// partials[block] (the state's table, or the library's device scratch) and an
// overflow flag.  A fold kernel adds the partials into st->sumsq in a fixed
// order, so the sum is reproducible.  The partials bound the grid (at most
// ZERO_MAX_PARTIALS blocks); a shard that needs more blocks is reduced in
// several launches over consecutive tile ranges, block b of every later
// launch adding its sum onto partials[b], so the fold still sees one fixed
// order.
//
// Mapping (quad, as the AdamW kernel): in chunk j of a tile, lane l owns
// elements 256j + 4l .. 4l+3, so every wave instruction covers one contiguous
// span (512 B of each 16-bit input, 1 KiB of the fp32 output); a lane stride
// that leaves half of each cache line to another instruction costs about a
// third of the bandwidth here.
//
// Work split: a launch covers full tiles [tile0, tile_end); wave w walks runs
// of R consecutive tiles from tile0 + w*R, then w*R + nwaves*R, ...  The
// launcher picks R (one tile per wave for the 16-bit and fp32 inputs, runs of
// about 16 steps for INT8 payloads) and sizes the grid so that each wave has
// one run.  The first launch of a shard also does the head elements, the last
// one the ragged tail.
//
// Pipelining: a wave walks (tile, group of KC buffers) pairs in order and
// issues the reads of the next pair before adding the current one and before
// storing a finished tile; a scheduling barrier keeps the compiler from sinking
// them.  KC divides N (chosen by the launcher), so no group is partial and the
// loop body has no per-buffer branches; G1 marks N == KC (one group).
//
// Sources: a RawQuad<DT> holds one lane's four inputs of one rank buffer as
// loaded (load) and adds their values to the accumulators (add_to); one()
// gives a single element for the ragged tail.  DT is the buffer format, or
// kQ8: INT8 codes with one fp32 scale per block (the quantised-gradient
// Reduce-Scatter payload), rank k's codes at bufs[2k] and scales at bufs[2k+1];
// its value is f32(code) * scale, one binary32 product.
constexpr int kQ8 = 3;

// reduce launch parts (the `part` argument)
constexpr int kPartFirst = 1;   // does the head elements (the shard's first launch)
constexpr int kPartLast = 2;    // does the ragged tail (its last launch)
constexpr int kPartAdd = 4;     // adds onto the partials of the launch before
constexpr int kPartFold = 8;    // one launch of at most kFoldThreads blocks: its last
                                // block folds the partials (no fold kernel)
constexpr int kFoldThreads = 1024;   // fold_kernel's block (one partial per thread and pass)
constexpr int kFoldU = 8;            // fold_kernel's loads in flight per thread

__device__ __forceinline__ int64_t block_of(const ReduceLaunch& a, int64_t i) {
    return a.block_shift >= 0 ? (i >> a.block_shift) : i / a.block;
}

// p + e0 + off, for a wave-uniform tile start e0 and a small per-lane element
// offset: the compiler keeps p + e0 in scalar registers and the lane's 32-bit
// byte offset in one vector register (the scalar-base addressing form), so no
// lane holds a 64-bit address per buffer.
template <typename T>
__device__ __forceinline__ T* lane_ptr(T* p, int64_t e0, uint32_t off) {
    typedef typename std::conditional<std::is_const<T>::value, const char, char>::type Byte;
    return reinterpret_cast<T*>(reinterpret_cast<Byte*>(p + e0) + off * (uint32_t)sizeof(T));
}

// Four consecutive elements of one rank's buffer at tile start e0 + lane
// offset off (elements).
template <int DT>
struct RawQuad;
template <>
struct RawQuad<ZERO_F32> {
    v4f x;
    __device__ __forceinline__ void load_ptr(const float* p, int64_t e0, uint32_t off) {
        x = ldnt_f4(lane_ptr(p, e0, off));
    }
    __device__ __forceinline__ void load(const ReduceLaunch& a, int k, int64_t e0, uint32_t off,
                                         int64_t) {
        load_ptr(static_cast<const float*>(a.bufs[k]), e0, off);
    }
    __device__ __forceinline__ void add_to(float acc[4]) const {
        acc[0] = acc[0] + x.x; acc[1] = acc[1] + x.y; acc[2] = acc[2] + x.z; acc[3] = acc[3] + x.w;
    }
    __device__ static __forceinline__ float one(const ReduceLaunch& a, int k, int64_t i) {
        return static_cast<const float*>(a.bufs[k])[i];
    }
};
template <>
struct RawQuad<kQ8> {
    uint32_t w;  // four codes
    float s;     // their block's scale (4 | block: a quad never straddles blocks)
    // bi: the block of the quad, the same for every rank (computed once per chunk)
    __device__ __forceinline__ void load(const ReduceLaunch& a, int k, int64_t e0, uint32_t off,
                                         int64_t bi) {
        w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
            lane_ptr(static_cast<const int8_t*>(a.bufs[2 * k]), e0, off)));
        s = static_cast<const float*>(a.bufs[2 * k + 1])[bi];
    }
    __device__ __forceinline__ void add_to(float acc[4]) const {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[c] = acc[c] + (float)((int32_t)(w << (24 - 8 * c)) >> 24) * s;
    }
    __device__ static __forceinline__ float one(const ReduceLaunch& a, int k, int64_t i) {
        return (float)static_cast<const int8_t*>(a.bufs[2 * k])[i] *
               static_cast<const float*>(a.bufs[2 * k + 1])[block_of(a, i)];
    }
};
template <int DT>
struct RawQuad {
    v2u w;
    __device__ __forceinline__ void load(const ReduceLaunch& a, int k, int64_t e0, uint32_t off,
                                         int64_t) {
        w = ldnt_u2(lane_ptr(static_cast<const uint16_t*>(a.bufs[k]), e0, off));
    }
    __device__ __forceinline__ void add_to(float acc[4]) const {
        acc[0] = acc[0] + cvt16<DT>(w.x & 0xffffu);
        acc[1] = acc[1] + cvt16<DT>(w.x >> 16);
        acc[2] = acc[2] + cvt16<DT>(w.y & 0xffffu);
        acc[3] = acc[3] + cvt16<DT>(w.y >> 16);
    }
    __device__ static __forceinline__ float one(const ReduceLaunch& a, int k, int64_t i) {
        return cvt16<DT>(static_cast<const uint16_t*>(a.bufs[k])[i]);
    }
};

// Shifted slices (SHIFT): the rank slices do not start on a 128-byte line
// (rank r's slice starts at r*S of its buffer, for any S), while the fp32
// output is aligned.  The first `head` elements (up to the slices' next line
// boundary) go element-wise; the tiles then read whole lines of every slice,
// from element head on.  Tile t's input elements head + t*T + i land on the
// output at hq + t*T + i + sh, with hq = head - sh a multiple of 4 and
// sh = head % 4: the reduced quads are computed in the input lane layout and,
// when sh != 0, one cross-lane shift per chunk turns them into aligned output
// quads -- output position D takes input position D - sh of its own lane, or
// D - sh + 4 of the lane below.  Then the output quad at each tile start is
// shared with the tile below, and each tile writes its part of it (and of
// the next tile's first quad) element-wise.  Reading partial lines instead
// (tiles starting at the first quad-aligned element) fetched each tile's edge
// lines twice: 18% slower on the 8-slice reduce, 40% on the statistics pass.
// The value lane l - 1 holds (lane 0: its own): one DPP wave shift right by one
// lane (a gfx9-family DPP control), no LDS crossbar traffic.
constexpr int kDppWaveShr1 = 0x138;
__device__ __forceinline__ float from_lane_below(float x) {
    const int v = __float_as_int(x);
    return __int_as_float(__builtin_amdgcn_update_dpp(v, v, kDppWaveShr1, 0xf, 0xf, false));
}
// The value lane 63 holds, in every lane (a scalar read of one lane).
__device__ __forceinline__ float from_last_lane(float x) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ uint32_t lane_below_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppWaveShr1, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t last_lane_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

template <int D>
__device__ __forceinline__ float shift_pick(int sh, const float (&mine)[4], const float (&up)[4]) {
    const float a1 = D >= 1 ? mine[(D + 3) & 3] : up[3];
    const float a2 = D >= 2 ? mine[(D + 2) & 3] : up[(D + 2) & 3];
    const float a3 = D >= 3 ? mine[0] : up[(D + 1) & 3];
    return sh == 0 ? mine[D] : (sh == 1 ? a1 : (sh == 2 ? a2 : a3));
}

template <int DT, bool VEC, bool SHIFT, bool WRITE, bool STATS, int TU, int KC, bool ACC, bool G1>
__global__ void __launch_bounds__(kThreads) reduce_kernel(ReduceLaunch a, float inv_n,
                                                          int pow2_n, int run_tiles,
                                                          int64_t tile0, int64_t tile_end,
                                                          int part) {
    static_assert(WRITE || !ACC, "accumulation writes its output");
    static_assert(VEC || !SHIFT, "the shifted layout is a vector layout");
    static_assert(DT != kQ8 || !SHIFT, "INT8 payload slices are not shifted");
    constexpr int64_t kT = 256 * TU;
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t n = a.n;
    const int N = a.n_ranks;
    const int ngroups = G1 ? 1 : N / KC;   // G1: the N buffers form one group
    const bool avg = a.op == ZERO_AVG;
    float inv_scale = 1.0f;
    if constexpr (STATS) inv_scale = (float)(1.0 / (double)a.st->loss_scale);
    const float fN = (float)N;

    // Sum of u^2 in two fixed-order binary64 chains (elements 0,1 / 2,3 of
    // each quad).  u*u is exact in binary64, so fma(u, u, s) equals s + u*u
    // rounded once.  No term can overflow binary64 (|u| < 2^128) and squares
    // are >= 0, so the sum is non-finite exactly when some u is inf or NaN:
    // that is the overflow test, taken once per lane after the loop.
    double ss0 = 0.0, ss1 = 0.0;

    // SHIFT: head elements before the slices' first line boundary, their shift
    // within an output quad and the (quad-aligned) output offset of tile 0
    const int64_t hs = SHIFT ? a.head : 0;
    const int sh = (int)(hs & 3);
    const int64_t hq = hs - sh;
    // the reduce (AVG applied) of one element from its rank-order sum
    auto reduced = [&](float sum) -> float {
        const float q = pow2_n ? sum * inv_n : sum / fN;
        return avg ? q : sum;
    };
    // one element written on its own: value r (reduced), pv its accumulated
    // value (ACC)
    auto put_one = [&](int64_t i, float r, float pv) {
        float val = r;
        if constexpr (ACC) val = pv + r;
        if constexpr (WRITE) a.red_out[i] = val;
        if constexpr (STATS) {
            const double u = (double)(val * inv_scale);
            ss0 = __builtin_fma(u, u, ss0);
        }
    };

    const int64_t nbody = n > hs ? n - hs : 0;       // elements from the slices' first line boundary on
    const int64_t ntiles = (nbody + kT - 1) / kT;
    const int64_t nfull = VEC ? nbody / kT : 0;
    // SHIFT: lane 63's reduced values of the last chunk of the tile this wave
    // finished last; when the wave's next tile follows it (inside a run of
    // consecutive tiles) they complete that tile's first output quad, so the
    // quads shared between tiles are split only at the ends of a run.
    float run_carry[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t R = run_tiles;
    // prev: the shard's accumulated values for these elements (ACC only)
    // the quads of the tile at e0 that this lane owns start at e0 + lo + 256 j
    auto finish = [&](const float (&acc)[TU][4], const float (&prev)[TU][4], int64_t e0,
                      uint32_t lo, bool full) {
        if constexpr (SHIFT) {
            if (full && !WRITE) {
                // statistics only: every element of the tile is this lane's, in
                // the input layout; nothing to place on an output
#pragma unroll
                for (int j = 0; j < TU; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const double u = (double)(reduced(acc[j][c]) * inv_scale);
                        if (c & 2) ss1 = __builtin_fma(u, u, ss1);
                        else ss0 = __builtin_fma(u, u, ss0);
                    }
                return;
            }
            if (full) {
                // acc holds input elements e0 + sh + 256j + lo + c; output quad
                // (j, lane) is e0 + 256j + lo + d, and prev holds it (ACC);
                // e0 = hq + t*T
                const int64_t tt = (e0 - hq) / kT;
                const bool after = (tt - tile0) % R != 0;                  // the tile below was this wave's
                const bool before = (tt + 1 - tile0) % R != 0 && tt + 1 < tile_end;  // and so is the next
                float carry[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) carry[c] = run_carry[c];
#pragma unroll
                for (int j = 0; j < TU; ++j) {
                    float mine[4], up[4], out[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) mine[c] = reduced(acc[j][c]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) up[c] = from_lane_below(mine[c]);
                    if ((j > 0 || after) && lane == 0) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) up[c] = carry[c];
                    }
                    out[0] = shift_pick<0>(sh, mine, up);
                    out[1] = shift_pick<1>(sh, mine, up);
                    out[2] = shift_pick<2>(sh, mine, up);
                    out[3] = shift_pick<3>(sh, mine, up);
#pragma unroll
                    for (int c = 0; c < 4; ++c) carry[c] = from_last_lane(mine[c]);
                    const int64_t o0 = e0 + lo + 256 * j;
                    if (sh != 0 && j == 0 && !after && lane == 0) {
                        // the first sh elements of this quad belong to another wave's tile
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            if (d >= sh) put_one(o0 + d, out[d], prev[0][d]);
                    } else {
                        float val[4];
#pragma unroll
                        for (int d = 0; d < 4; ++d) val[d] = ACC ? prev[j][d] + out[d] : out[d];
                        stnt_f4(lane_ptr(a.red_out, e0, lo + 256 * j), val[0], val[1], val[2], val[3]);
                        if constexpr (STATS) {
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                const double u = (double)(val[d] * inv_scale);
                                if (d & 2) ss1 = __builtin_fma(u, u, ss1);
                                else ss0 = __builtin_fma(u, u, ss0);
                            }
                        }
                    }
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) run_carry[c] = carry[c];
                // the last lane's top elements open the next tile's first quad:
                // stored here unless this wave finishes that tile next
                if (!before && lane == 0) {
#pragma unroll
                    for (int d = 0; d < 3; ++d) {
                        if (d < sh) {
                            const int64_t i = e0 + kT + d;
                            const int c = d + 4 - sh;
                            const float r = c == 1 ? carry[1] : (c == 2 ? carry[2] : carry[3]);
                            put_one(i, r, ACC ? a.red_out[i] : 0.0f);
                        }
                    }
                }
                return;
            }
        }
#pragma unroll
        for (int j = 0; j < TU; ++j) {
            const int64_t i0 = e0 + lo + 256 * j;
            float red[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float q = pow2_n ? acc[j][c] * inv_n : acc[j][c] / fN;
                red[c] = avg ? q : acc[j][c];
                if constexpr (ACC) red[c] = prev[j][c] + red[c];
            }
            if constexpr (WRITE) {
                if (full) {
                    stnt_f4(lane_ptr(a.red_out, e0, lo + 256 * j), red[0], red[1], red[2], red[3]);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (i0 + c < n) a.red_out[i0 + c] = red[c];
                }
            }
            if constexpr (STATS) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (full || i0 + c < n) {
                        const double u = (double)(red[c] * inv_scale);
                        if (c & 2) ss1 = __builtin_fma(u, u, ss1);
                        else ss0 = __builtin_fma(u, u, ss0);
                    }
                }
            }
        }
    };

    // ---- full tiles.  A step is one (tile, buffer group) pair.  Wave w walks
    // runs of R consecutive tiles: run w, then run w + nwaves, ...; inside a
    // tile it walks the buffer groups in rank order.
    //
    // Software pipeline: the next step's reads are issued before the current
    // step's adds and stores.  Two register sets A and B swap roles every
    // step (the loop body is a pair of steps), so no register copy has to
    // wait for reads in flight.  The wave's step count is known up front, so
    // the loop body holds no exit and no conditional read; the last one or
    // two steps run after it.  The compiler then waits for exactly the reads
    // the adds need and keeps the next step's reads (and earlier stores) in
    // flight.
    const int64_t wt0 = tile0 + wave_id * R;            // this wave's first full tile
    if (wt0 < tile_end) {
        RawQuad<DT> xa[KC][TU], xb[KC][TU];
        RawQuad<ZERO_F32> pa[TU], pb[TU];   // accumulator quads (ACC only)
        const uint32_t lo = 4 * lane;
        auto load_group = [&](RawQuad<DT> (&x)[KC][TU], RawQuad<ZERO_F32> (&px)[TU], int64_t tt,
                              int gg) {
            const int64_t e0 = tt * kT + hq;              // the output quads' tile start
            const int64_t ei = tt * kT + hs;              // the inputs' tile start
            int64_t bi[TU];
#pragma unroll
            for (int j = 0; j < TU; ++j) bi[j] = DT == kQ8 ? block_of(a, ei + lo + 256 * j) : 0;
#pragma unroll
            for (int kk = 0; kk < KC; ++kk)
#pragma unroll
                for (int j = 0; j < TU; ++j) x[kk][j].load(a, gg * KC + kk, ei, lo + 256 * j, bi[j]);
            if constexpr (ACC) {   // the shard's values, with the group that finishes the tile
                if (G1 || gg == ngroups - 1) {
#pragma unroll
                    for (int j = 0; j < TU; ++j) px[j].load_ptr(a.red_out, e0, lo + 256 * j);
                }
            }
        };
        float acc[TU][4];
#pragma unroll
        for (int j = 0; j < TU; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[j][c] = 0.0f;
        // add the group held in x; the tile's last group also finishes it
        auto consume = [&](const RawQuad<DT> (&x)[KC][TU], const RawQuad<ZERO_F32> (&px)[TU],
                           int64_t tt, int gg) {
#pragma unroll
            for (int kk = 0; kk < KC; ++kk)                  // rank order per element
#pragma unroll
                for (int j = 0; j < TU; ++j) x[kk][j].add_to(acc[j]);
            if (G1 || gg == ngroups - 1) {
                float prev[TU][4];
#pragma unroll
                for (int j = 0; j < TU; ++j) {
                    prev[j][0] = px[j].x.x; prev[j][1] = px[j].x.y;
                    prev[j][2] = px[j].x.z; prev[j][3] = px[j].x.w;
                }
                finish(acc, prev, tt * kT + hq, lo, true);
#pragma unroll
                for (int j = 0; j < TU; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[j][c] = 0.0f;
            }
        };
        // this wave's full tiles: runs start at w*R + j*nwaves*R; every run
        // but the last holds R tiles
        const int64_t span = nwaves * R;
        const int64_t q = tile_end - wt0;                 // > 0 here
        const int64_t runs = (q + span - 1) / span;
        const int64_t last = q - (runs - 1) * span;
        const int64_t nsteps = ((runs - 1) * R + (last < R ? last : R)) * ngroups;
        int64_t t = wt0, left = R;
        int g = 0;
        auto advance = [&]() {   // (t, g) := the step after (t, g)
            ++g;
            if (G1 || g == ngroups) {
                g = 0;
                if (left == 1) {
                    t += 1 + (nwaves - 1) * R;
                    left = R;
                } else {
                    t += 1;
                    --left;
                }
            }
        };
        load_group(xa, pa, t, g);
        int64_t k = 0;                                    // A holds step k
        for (; k + 2 < nsteps; k += 2) {                  // steps k+1 and k+2 exist
            const int64_t t0 = t;
            const int g0 = g;
            advance();
            load_group(xb, pb, t, g);
            __builtin_amdgcn_sched_barrier(0);
            consume(xa, pa, t0, g0);
            const int64_t t1 = t;
            const int g1 = g;
            advance();
            load_group(xa, pa, t, g);
            __builtin_amdgcn_sched_barrier(0);
            consume(xb, pb, t1, g1);
        }
        if (k + 1 < nsteps) {                             // two steps left
            const int64_t t0 = t;
            const int g0 = g;
            advance();
            load_group(xb, pb, t, g);
            __builtin_amdgcn_sched_barrier(0);
            consume(xa, pa, t0, g0);
            consume(xb, pb, t, g);
        } else {
            consume(xa, pa, t, g);
        }
    }
    // ---- the head (SHIFT): the elements before the slices' first line boundary
    if constexpr (SHIFT) {
        if ((part & kPartFirst) && wave_id == 0 && lane < hs && lane < n) {
            float sum = 0.0f;
            for (int k = 0; k < N; ++k) sum = sum + RawQuad<DT>::one(a, k, lane);
            put_one(lane, reduced(sum), ACC ? a.red_out[lane] : 0.0f);
        }
    }
    // ---- the ragged tail (or every tile, without the vector path): element-wise
    for (int64_t t = nfull + wave_id; (part & kPartLast) && t < ntiles; t += nwaves) {
        const int64_t base = hs + t * kT + 4 * lane;
        float acc[TU][4];
#pragma unroll
        for (int j = 0; j < TU; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[j][c] = 0.0f;
        for (int k = 0; k < N; ++k) {
#pragma unroll
            for (int j = 0; j < TU; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t i = base + 256 * j + c;
                    if (i < n) acc[j][c] = acc[j][c] + RawQuad<DT>::one(a, k, i);
                }
        }
        float prev[TU][4];
#pragma unroll
        for (int j = 0; j < TU; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t i = base + 256 * j + c;
                prev[j][c] = (ACC && i < n) ? a.red_out[i] : 0.0f;
            }
        finish(acc, prev, hs + t * kT, 4 * lane, false);
    }
    if constexpr (STATS) {
        const double mine = ss0 + ss1;
        const int ovf = !isfinite(mine);
        const double bs = block_sum(mine);
        if (threadIdx.x == 0) {
            if (part & kPartAdd) {
                a.partials[blockIdx.x] = a.partials[blockIdx.x] + bs;
            } else {
                a.partials[blockIdx.x] = bs;
                if (blockIdx.x == 0) a.st->n_partials = (int32_t)gridDim.x;
            }
        }
        if (__ballot(ovf) != 0ull && lane == 0) atomicOr(&a.st->overflow, 1);
        if (part & kPartFold) {
            // A small reduce folds its own partials: each block counts itself
            // in after its partial (device-scope release), and the block that
            // counts last (acquire) adds them in fold_kernel's order -- virtual
            // thread t of 1024 holds partial t (or +0), each virtual wave's
            // butterfly, then the 16 wave sums in order -- so st->sumsq gets the
            // same bits as from the fold kernel.  The count lives in the state's
            // counter field and is returned to zero here.
            __shared__ int s_last;
            __shared__ double s_wave[kFoldThreads / 64];
            unsigned* count = reinterpret_cast<unsigned*>(&a.st->tile_counter);
            if (threadIdx.x == 0) {
                __threadfence();
                s_last = atomicAdd(count, 1u) == gridDim.x - 1;
            }
            __syncthreads();
            if (s_last) {
                __threadfence();
                const int np = (int)gridDim.x;
                for (int vw = (int)(threadIdx.x >> 6); vw < kFoldThreads / 64; vw += kWaves) {
                    const int i = vw * 64 + lane;
                    double x = 0.0;
                    if (i < np) x = x + a.partials[i];
                    x = wave_sum(x);
                    if (lane == 0) s_wave[vw] = x;
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    double t = 0.0;
#pragma unroll
                    for (int w = 0; w < kFoldThreads / 64; ++w) t += s_wave[w];
                    a.st->sumsq = a.st->sumsq + t;
                    atomicExch(count, 0u);
                }
            }
        }
    }
}

// st->sumsq += partials[0..n_partials), fixed order (one block); partials is
// the state's own table, or the library's device scratch (the no-allocation
// reduce entry point)
// One block of kFoldThreads: thread t adds partials t, t + kFoldThreads, ...
// in that order, with kFoldU loads in flight (an out-of-range slot adds +0,
// which leaves a sum of non-negative terms unchanged); then the waves'
// butterflies and the waves in index order.
__global__ void __launch_bounds__(kFoldThreads) fold_kernel(zero_step_state_t* st,
                                                            const double* partials) {
    const int n = st->n_partials;
    double s = 0.0;
    for (int i0 = threadIdx.x; i0 < n; i0 += kFoldThreads * kFoldU) {
        double v[kFoldU];
#pragma unroll
        for (int u = 0; u < kFoldU; ++u) {
            const int i = i0 + u * kFoldThreads;
            v[u] = i < n ? partials[i] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kFoldU; ++u) s += v[u];
    }
    __shared__ double sh[kFoldThreads / 64];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kFoldThreads / 64; ++w) t += sh[w];
        st->sumsq = st->sumsq + t;
    }
}

// ---------------------------------------------------------------- INT8 of one slice
// x[4]: this lane's four written values (zero for elements past the end).
// One 256-element block per wave slice: amax across the wave, then codes.
//
// The code is rint(x / scale) with the IEEE quotient, whose division sequence
// dominates this function.  The quotient is first taken as y = x * (1/scale)
// (two roundings): that is within |q| * 2^-22 of the IEEE quotient q, and
// |q| <= 127.0002 here (|x| <= amax, scale = amax/127 rounded), so within
// 2^-15, and both round to the same integer unless y lies within 2^-15 of a
// half-integer.  Elements within 2^-14 of one (about one in 8000) take the
// exact division, in a branch the whole wave skips when no lane needs it; so
// does every element when 1/scale is infinite or zero (scale below 2^-128, or
// infinite).
__device__ __forceinline__ uint32_t quant_quad(const float x[4], float* scale_out) {
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) a = fmaxf(a, fabsf(x[c]));
    const float amax = wave_max(a);
    const float scale = amax / 127.0f;
    const float rs = 1.0f / scale;
    const bool fast = isfinite(rs) && rs != 0.0f;
    float r[4];
    bool exact[4];
    bool any = false;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float y = x[c] * rs;
        const float f = y - floorf(y);                  // the fraction, within 2^-24
        exact[c] = !fast || fabsf(f - 0.5f) <= 0x1p-14f;  // NaN y: not near, rint gives NaN
        r[c] = rintf(y);
        any = any || exact[c];
    }
    if (__any(any)) {                                   // wave-uniform
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (exact[c]) r[c] = rintf(x[c] / scale);  // ties to even
    }
    uint32_t packed = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float v = 0.0f;
        if (amax != 0.0f) {
            v = isnan(r[c]) ? 0.0f : r[c];
            v = fminf(fmaxf(v, -127.0f), 127.0f);
        }
        packed |= ((uint32_t)(int32_t)v & 0xffu) << (8 * c);
    }
    *scale_out = scale;
    return packed;
}

// ---------------------------------------------------------------- AdamW
// The update of one lane's four elements, in the step's operation order:
// unscale, clip, the two moments, bias corrections, decoupled decay, then the
// 16-bit write-back value (its bits and the value the slot then holds).
template <int PT>
__device__ __forceinline__ void adam_quad_math(const AdamLaunch& a, const StepScalars& s,
                                               const float gv[4], float pv[4], float mv[4],
                                               float vv[4], uint32_t lp16[4], float lpv[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float uu = gv[c] * s.inv;      // unscale
        const float g = uu * s.coef;         // clip
        const float mn = a.b1 * mv[c] + a.c1 * g;
        const float vn = a.b2 * vv[c] + a.c2 * (g * g);
        const float mh = mn / s.bc1;
        const float vh = vn / s.bc2;
        const float d = sqrtf(vh) + a.eps;
        const float pn = pv[c] * a.wdf - (a.lr * mh) / d;
        pv[c] = pn;
        mv[c] = mn;
        vv[c] = vn;
        lp16[c] = round16<PT>(pn);
        lpv[c] = cvt16<PT>(lp16[c]);         // the value the slot now holds
    }
}

// A full tile: one buffer resource per array over the tile (wave-uniform
// bases in scalar registers, 32-bit lane offsets); every slice's loads are
// issued before any arithmetic.
//
// The slot and the INT8 codes may start anywhere (rank r's slot sits at r*S
// of the All-Gather buffer, for any S), while master/m/v and the gradient
// keep the vector layout.  Then each lane's four 16-bit values (four codes)
// are joined with the top of the lane below (one DPP wave shift) into the
// aligned word that covers them, so every store is a whole aligned word; the
// tile's first word is shared with the tile below and its last elements open
// the next tile's first word, and those few are stored element by element.
// Stores of whole 8-byte words at 2-byte offsets instead cost the update 5%.
template <int GT, int PT, bool QUANT>
__device__ __forceinline__ void adam_tile_full(const AdamLaunch& a, const StepScalars& s,
                                               int64_t base, int lane) {
    constexpr uint32_t ges = GT == ZERO_F32 ? 4 : 2;
    uint16_t* const lp = static_cast<uint16_t*>(a.lp);
    // the slot's (codes') start within an aligned 8-byte (4-byte) word, in elements
    const int ms = (int)((reinterpret_cast<uintptr_t>(lp) >> 1) & 3);
    const int mq = QUANT ? (int)(reinterpret_cast<uintptr_t>(a.q) & 3) : 0;
    const BufRes rg = buf_res(static_cast<const char*>(a.g) + base * ges, (uint32_t)(kTile * ges));
    const BufRes rp = buf_res(a.p + base, (uint32_t)(kTile * 4));
    const BufRes rm = buf_res(a.m + base, (uint32_t)(kTile * 4));
    const BufRes rv = buf_res(a.v + base, (uint32_t)(kTile * 4));
    // over the aligned words of the tile's slot (codes): word k at byte 8k (4k)
    const BufRes rl = buf_res(lp + base - ms, (uint32_t)(kTile * 2));
    float gv[kU][4], pv[kU][4], mv[kU][4], vv[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t e = 256 * u + 4 * lane;   // element offset within the tile
        bload_quad<GT>(rg, e * ges, gv[u]);
        bload_quad<ZERO_F32>(rp, e * 4, pv[u]);
        bload_quad<ZERO_F32>(rm, e * 4, mv[u]);
        bload_quad<ZERO_F32>(rv, e * 4, vv[u]);
    }
    uint32_t carry_lo = 0, carry_hi = 0, carry_q = 0;   // lane 63's words of the slice before
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t e = 256 * u + 4 * lane;
        uint32_t lp16[4];
        float lpv[4];
        adam_quad_math<PT>(a, s, gv[u], pv[u], mv[u], vv[u], lp16, lpv);
        bstore_f4(rp, e * 4, pv[u]);
        bstore_f4(rm, e * 4, mv[u]);
        bstore_f4(rv, e * 4, vv[u]);
        const uint32_t wlo = lp16[0] | (lp16[1] << 16), whi = lp16[2] | (lp16[3] << 16);
        if (ms == 0) {
            v2u w;
            w.x = wlo;
            w.y = whi;
            bst_u2(rl, e * 2, w);
        } else {
            uint32_t blo = lane_below_u(wlo), bhi = lane_below_u(whi);
            if (lane == 0) {
                blo = carry_lo;
                bhi = carry_hi;
            }
            const uint64_t mine = (uint64_t)wlo | ((uint64_t)whi << 32);
            const uint64_t below = (uint64_t)blo | ((uint64_t)bhi << 32);
            const uint64_t x = (mine << (16 * ms)) | (below >> (64 - 16 * ms));
            carry_lo = last_lane_u(wlo);
            carry_hi = last_lane_u(whi);
            if (u == 0 && lane == 0) {      // the word shared with the tile below
                for (int c = 0; c < 4 - ms; ++c) lp[base + c] = (uint16_t)lp16[c];
            } else {
                v2u w;
                w.x = (uint32_t)x;
                w.y = (uint32_t)(x >> 32);
                bst_u2(rl, e * 2, w);
            }
            if (u == kU - 1 && lane == 63) {   // the start of the next tile's first word
                for (int c = 4 - ms; c < 4; ++c) lp[base + e + c] = (uint16_t)lp16[c];
            }
        }
        if constexpr (QUANT) {
            float scale;
            const uint32_t q = quant_quad(lpv, &scale);  // whole wave takes part
            if (mq == 0) {
                bst_u1(buf_res(a.q + base, (uint32_t)kTile), e, q);
            } else {
                uint32_t b = lane_below_u(q);
                if (lane == 0) b = carry_q;
                const uint32_t x = (q << (8 * mq)) | (b >> (32 - 8 * mq));
                carry_q = last_lane_u(q);
                if (u == 0 && lane == 0) {
                    for (int c = 0; c < 4 - mq; ++c) a.q[base + c] = (int8_t)(q >> (8 * c));
                } else {
                    bst_u1(buf_res(a.q + base - mq, (uint32_t)kTile), e, x);
                }
                if (u == kU - 1 && lane == 63) {
                    for (int c = 4 - mq; c < 4; ++c) a.q[base + e + c] = (int8_t)(q >> (8 * c));
                }
            }
            if (lane == 0) a.qs[(base + 256 * u) / 256] = scale;
        }
    }
}

// The last, partial tile (or every tile when a pointer does not allow the
// vector accesses): element-wise, one slice at a time, so that it holds few
// registers (the kernel's register count is that of its largest path).
template <int GT, int PT, bool QUANT>
__device__ __forceinline__ void adam_tile_part(const AdamLaunch& a, const StepScalars& s,
                                               int64_t base, int lane) {
    const int64_t n = a.n;
    uint16_t* lp = static_cast<uint16_t*>(a.lp);
#pragma unroll 1
    for (int u = 0; u < kU; ++u) {
        const int64_t i0 = base + 256 * u + 4 * lane;
        float gv[4], pv[4], mv[4], vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool ok = i0 + c < n;
            gv[c] = ok ? load_one<GT>(a.g, i0 + c) : 0.0f;
            pv[c] = ok ? a.p[i0 + c] : 0.0f;
            mv[c] = ok ? a.m[i0 + c] : 0.0f;
            vv[c] = ok ? a.v[i0 + c] : 0.0f;
        }
        uint32_t lp16[4];
        float lpv[4];
        adam_quad_math<PT>(a, s, gv, pv, mv, vv, lp16, lpv);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (i0 + c < n) {
                a.p[i0 + c] = pv[c];
                a.m[i0 + c] = mv[c];
                a.v[i0 + c] = vv[c];
                lp[i0 + c] = (uint16_t)lp16[c];
            } else {
                lpv[c] = 0.0f;
            }
        }
        if constexpr (QUANT) {
            float scale;
            const uint32_t q = quant_quad(lpv, &scale);  // whole wave takes part
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (i0 + c < n) a.q[i0 + c] = (int8_t)((q >> (8 * c)) & 0xffu);
            const int64_t blk0 = base + 256 * u;
            if (lane == 0 && blk0 < n) a.qs[blk0 / 256] = scale;
        }
    }
}

template <int GT, int PT, bool QUANT, bool VEC>
__global__ void __launch_bounds__(kThreads) adamw_kernel(AdamLaunch a, int64_t t0, int64_t t1) {
    const StepScalars s = read_step(a.st, a.beta1, a.beta2, a.max_norm);
    if (s.skip) return;  // overflow on this or another rank: nothing is written
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t ntiles = (a.n + kTile - 1) / kTile;
    const int64_t nfull = VEC ? a.n / kTile : 0;
    for (int64_t t = t0 + wave_id; t < t1 && t < ntiles; t += nwaves) {
        if (t < nfull) adam_tile_full<GT, PT, QUANT>(a, s, t * kTile, lane);
        else adam_tile_part<GT, PT, QUANT>(a, s, t * kTile, lane);
    }
}

// The update of a large shard (with or without the INT8 epilogue): a
// persistent grid of two blocks per compute unit takes groups of kWaves
// consecutive tiles (one per wave) from a counter in the state, in the order
// the blocks ask, so the tiles in flight stay in one narrow window of every
// array however the XCDs drift (measured 0.6-2.8% faster than launch slices
// of 32,768 blocks on three allocations, at full occupancy 10% slower; with
// the INT8 epilogue 4% faster than full-occupancy slices on three of four
// allocations, 5% slower on the fourth, and within 1.3% across all four).
// Each tile is updated exactly once whichever block takes it, so the results
// do not depend on the order.  A block takes its next group while it updates
// the current one; every block's last request comes back past the end, so
// there are exactly ngroups + gridDim.x requests, and the block whose request
// is the last one returns the counter to zero for the next launch.  A skipped
// step takes no group and leaves the counter at zero.
template <int GT, int PT, bool QUANT>
__global__ void __launch_bounds__(kThreads) adamw_sched_kernel(AdamLaunch a) {
    const StepScalars s = read_step(a.st, a.beta1, a.beta2, a.max_norm);
    if (s.skip) return;
    unsigned* counter = reinterpret_cast<unsigned*>(&a.st->tile_counter);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t ntiles = (a.n + kTile - 1) / kTile;
    const int64_t nfull = a.n / kTile;
    const unsigned ngroups = (unsigned)((ntiles + kWaves - 1) / kWaves);
    __shared__ unsigned s_group;
    unsigned next = 0;
    if (threadIdx.x == 0) s_group = atomicAdd(counter, 1u);
    __syncthreads();
    unsigned g = s_group;
    __syncthreads();
    while (g < ngroups) {
        if (threadIdx.x == 0) next = atomicAdd(counter, 1u);
        const int64_t t = (int64_t)g * kWaves + w;
        if (t < nfull) adam_tile_full<GT, PT, QUANT>(a, s, t * kTile, lane);
        else if (t < ntiles) adam_tile_part<GT, PT, QUANT>(a, s, t * kTile, lane);
        if (threadIdx.x == 0) s_group = next;
        __syncthreads();
        g = s_group;
        __syncthreads();
    }
    if (threadIdx.x == 0 && g == ngroups + gridDim.x - 1) atomicExch(counter, 0u);
}

// Loss scaler and counters after the step (one thread).
__global__ void finalize_kernel(zero_step_state_t* st, double beta1, double beta2,
                                double max_norm) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const StepScalars s = read_step(st, beta1, beta2, max_norm);
    st->last_norm = sqrt(st->sumsq + st->remote_sumsq);
    st->last_skipped = s.skip;
    st->last_coef = s.skip ? 0.0f : s.coef;
    if (s.skip) {
        if (st->dynamic) {
            const float h = st->loss_scale / 2.0f;
            st->loss_scale = h > st->min_scale ? h : st->min_scale;
        }
        st->good_steps = 0;
    } else {
        st->step = st->step + 1;
        st->beta1_pow = st->beta1_pow * beta1;
        st->beta2_pow = st->beta2_pow * beta2;
        if (st->dynamic) {
            st->good_steps = st->good_steps + 1;
            if (st->good_steps == st->window) {
                // doubling stops at 2^127 (the largest binary32 power of two), so
                // the scale and its reciprocal stay finite and exact
                if (st->loss_scale < 0x1p127f) st->loss_scale = st->loss_scale * 2.0f;
                st->good_steps = 0;
            }
        }
    }
    st->sumsq = 0.0;
    st->overflow = 0;
}

// ---------------------------------------------------------------- standalone INT8
template <int DT, bool VEC>
__global__ void __launch_bounds__(kThreads) quant_kernel(QuantLaunch a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t n = a.n;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    const int64_t nfull = VEC ? n / kTile : 0;
    for (int64_t t = wave_id; t < ntiles; t += nwaves) {
        const bool full = t < nfull;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i0 = t * kTile + 256 * u + 4 * lane;
            float x[4];
            if (full) {
                load_quad<DT>(a.x, i0, x);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) x[c] = i0 + c < n ? load_one<DT>(a.x, i0 + c) : 0.0f;
            }
            float scale;
            const uint32_t q = quant_quad(x, &scale);
            if (full) {
                stnt_u1(a.q + i0, q);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (i0 + c < n) a.q[i0 + c] = (int8_t)((q >> (8 * c)) & 0xffu);
            }
            const int64_t blk0 = t * kTile + 256 * u;
            if (lane == 0 && blk0 < n) a.qs[blk0 / 256] = scale;
        }
    }
}

// Standalone INT8 of a 16-bit slot with a lane mapping of its own (the AdamW
// epilogue keeps the quad mapping of the update): a wave tile is kQChunks
// chunks of 512 elements, and in each chunk lane l holds elements 8l .. 8l+7,
// one 16-byte load of 16-bit values and one 8-byte store of codes; every wave
// instruction still covers one contiguous span (1 KiB in, 512 B out).  Lanes
// 0-31 then hold one 256-element block and lanes 32-63 the next, so a block's
// absmax is a 5-step butterfly inside each half wave (against 6 steps per
// four elements in the quad mapping).  The per-element arithmetic is
// quant_quad's, so the codes and scales are the same bit for bit.
constexpr int kQChunks = 4;
constexpr int64_t kQTile = 512 * kQChunks;

__device__ __forceinline__ float half_wave_max(float x) {
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// x[8]: this lane's eight values (zero past the end); codes packed four per
// word into out[0..1]; the block's scale into *scale_out
__device__ __forceinline__ void quant_oct(const float x[8], uint32_t out[2], float* scale_out) {
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaxf(a, fabsf(x[c]));
    const float amax = half_wave_max(a);
    const float scale = amax / 127.0f;
    const float rs = 1.0f / scale;
    const bool fast = isfinite(rs) && rs != 0.0f;
    float r[8];
    bool exact[8];
    bool any = false;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float y = x[c] * rs;
        const float f = y - floorf(y);
        exact[c] = !fast || fabsf(f - 0.5f) <= 0x1p-14f;
        r[c] = rintf(y);
        any = any || exact[c];
    }
    if (__any(any)) {                                   // wave-uniform
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (exact[c]) r[c] = rintf(x[c] / scale);
    }
    out[0] = 0;
    out[1] = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float v = 0.0f;
        if (amax != 0.0f) {
            v = isnan(r[c]) ? 0.0f : r[c];
            v = fminf(fmaxf(v, -127.0f), 127.0f);
        }
        out[c >> 2] |= ((uint32_t)(int32_t)v & 0xffu) << (8 * (c & 3));
    }
    *scale_out = scale;
}

// x 16-byte aligned, q 8-byte aligned (checked by the host)
template <int DT>
__global__ void __launch_bounds__(kThreads) quant8_kernel(QuantLaunch a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t n = a.n;
    const int64_t ntiles = (n + kQTile - 1) / kQTile;
    const int64_t nfull = n / kQTile;
    const uint32_t lo = 8 * lane;
    const uint16_t* x16 = static_cast<const uint16_t*>(a.x);
    for (int64_t t = wave_id; t < ntiles; t += nwaves) {
        const int64_t e0 = t * kQTile;
        if (t < nfull) {
            v4u w[kQChunks];
#pragma unroll
            for (int k = 0; k < kQChunks; ++k)
                w[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u*>(lane_ptr(x16, e0 + 512 * k, lo)));
#pragma unroll
            for (int k = 0; k < kQChunks; ++k) {
                float x[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    x[2 * c] = cvt16<DT>(w[k][c] & 0xffffu);
                    x[2 * c + 1] = cvt16<DT>(w[k][c] >> 16);
                }
                uint32_t code[2];
                float scale;
                quant_oct(x, code, &scale);
                stnt_u2(lane_ptr(a.q, e0 + 512 * k, lo), code[0], code[1]);
                if ((lane & 31) == 0) a.qs[(e0 + 512 * k + lo) / 256] = scale;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kQChunks; ++k) {
                const int64_t i0 = e0 + 512 * k + lo;
                float x[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) x[c] = i0 + c < n ? load_one<DT>(a.x, i0 + c) : 0.0f;
                uint32_t code[2];
                float scale;
                quant_oct(x, code, &scale);               // the whole wave takes part
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (i0 + c < n) a.q[i0 + c] = (int8_t)((code[c >> 2] >> (8 * (c & 3))) & 0xffu);
                if ((lane & 31) == 0 && i0 < n) a.qs[i0 / 256] = scale;
            }
        }
    }
}

// ---------------------------------------------------------------- INT8 consumer
// out[s*S + i] = round(f32(q) * scale of (slot s, block i / block)).  A wave
// tile is kDU slices of 256 elements of one slot (tiles never straddle slots,
// so blocks restart at every slot start as the producer wrote them); in slice
// u lane l owns elements 256u + 4l .. 4l+3: one 4-byte code load, one 8-byte
// (16-bit) or 16-byte (fp32) store, each wave instruction one contiguous span.
// The scale is a cached load shared by the lanes of a block.
constexpr int kDU = 8;
constexpr int64_t kDTile = 256 * kDU;

template <int OT>
__device__ __forceinline__ void store_out_quad(void* out, int64_t i, const float x[4]) {
    if constexpr (OT == ZERO_F32) {
        stnt_f4(static_cast<float*>(out) + i, x[0], x[1], x[2], x[3]);
    } else {
        stnt_u2(static_cast<uint16_t*>(out) + i, round16<OT>(x[0]) | (round16<OT>(x[1]) << 16),
                round16<OT>(x[2]) | (round16<OT>(x[3]) << 16));
    }
}
template <int OT>
__device__ __forceinline__ void store_out_one(void* out, int64_t i, float x) {
    if constexpr (OT == ZERO_F32) static_cast<float*>(out)[i] = x;
    else static_cast<uint16_t*>(out)[i] = (uint16_t)round16<OT>(x);
}
// code c (0..3) of a little-endian 4-code word, sign-extended
__device__ __forceinline__ float code_of(uint32_t w, int c) {
    return (float)((int32_t)(w << (24 - 8 * c)) >> 24);
}

template <int OT, bool VEC>
__global__ void __launch_bounds__(kThreads) dequant_kernel(DequantLaunch a, int block_shift) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t S = a.slot_numel;
    const int64_t per_slot = (S + kDTile - 1) / kDTile;
    const int64_t ntiles = per_slot * a.n_slots;
    const int64_t nb = (S + a.block - 1) / a.block;
    auto block_of = [&](int64_t i) -> int64_t {
        return block_shift >= 0 ? (i >> block_shift) : i / a.block;
    };
    for (int64_t t = wave_id; t < ntiles; t += nwaves) {
        const int64_t slot = t / per_slot;
        const int64_t w0 = (t - slot * per_slot) * kDTile;  // first element within the slot
        const int8_t* q = a.q + slot * S;
        const float* qs = a.qs + slot * nb;
        const int64_t o0 = slot * S;
        if (VEC && w0 + kDTile <= S) {
            uint32_t code[kDU];
            float sc[kDU];
#pragma unroll
            for (int u = 0; u < kDU; ++u) {
                const int64_t i = w0 + 256 * u + 4 * lane;
                code[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q + i));
                sc[u] = qs[block_of(i)];                 // 4 | block: one block per lane quad
            }
#pragma unroll
            for (int u = 0; u < kDU; ++u) {
                float x[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) x[c] = code_of(code[u], c) * sc[u];
                store_out_quad<OT>(a.out, o0 + w0 + 256 * u + 4 * lane, x);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kDU; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t i = w0 + 256 * u + 4 * lane + c;
                    if (i < S) store_out_one<OT>(a.out, o0 + i, (float)q[i] * qs[block_of(i)]);
                }
        }
    }
}

// The same consumer with tiles laid over the flat output instead of each slot:
// every tile starts at a multiple of kDTile elements of the flat buffer, so a
// tile's stores cover whole cache lines of the output (and its code loads
// whole lines of the payload) whatever the slot size.  Tiled per slot, a slot
// size that is not a multiple of the 128-byte line left every tile edge
// splitting a line between two waves, and the counters showed those lines
// written back in two parts (4-6% extra bytes on such sizes, none on aligned
// ones).  Needs slot_numel >= kDTile (at most one slot boundary per tile) and
// the quad path (slot_numel % 4 == 0: a lane quad never straddles a slot or a
// block).
template <int OT>
__global__ void __launch_bounds__(kThreads) dequant_flat_kernel(DequantLaunch a, int block_shift,
                                                                int64_t t0, int64_t t1) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = wave_index();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t S = a.slot_numel;
    const int64_t total = S * a.n_slots;
    const int64_t nb = (S + a.block - 1) / a.block;
    const int64_t nfull = total / kDTile;
    const int64_t ntiles = (total + kDTile - 1) / kDTile;
    auto block_of = [&](int64_t i) -> int64_t {
        return block_shift >= 0 ? (i >> block_shift) : i / a.block;
    };
    for (int64_t t = t0 + wave_id; t < t1 && t < ntiles; t += nwaves) {
        const int64_t e0 = t * kDTile;
        const int64_t s0 = e0 / S;          // slot of the tile's first element
        const int64_t b1 = (s0 + 1) * S;    // first element of the next slot
        // the scale of the block holding flat element i (slot s0 or s0 + 1)
        auto scale_of = [&](int64_t i) -> float {
            const int64_t sl = i >= b1 ? s0 + 1 : s0;
            return a.qs[sl * nb + block_of(i - sl * S)];
        };
        if (t < nfull) {
            uint32_t code[kDU];
            float sc[kDU];
#pragma unroll
            for (int u = 0; u < kDU; ++u) {
                const int64_t i = e0 + 256 * u + 4 * lane;
                code[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.q + i));
                sc[u] = scale_of(i);                 // 4 | S and 4 | block: one block per quad
            }
#pragma unroll
            for (int u = 0; u < kDU; ++u) {
                float x[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) x[c] = code_of(code[u], c) * sc[u];
                store_out_quad<OT>(a.out, e0 + 256 * u + 4 * lane, x);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kDU; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t i = e0 + 256 * u + 4 * lane + c;
                    if (i < total) store_out_one<OT>(a.out, i, (float)a.q[i] * scale_of(i));
                }
        }
    }
}

// ---------------------------------------------------------------- launch helpers
// compute units of the current device, looked up once per device
constexpr int kMaxCuDevices = 64;
std::atomic<int> g_cu_count[kMaxCuDevices];

int cu_count_for_current_device(int* out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxCuDevices) return (int)hipErrorInvalidDevice;
    int n = g_cu_count[dev].load(std::memory_order_acquire);
    if (n <= 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return (int)e;
        if (n <= 0) return (int)hipErrorInvalidDevice;
        g_cu_count[dev].store(n, std::memory_order_release);
    }
    *out = n;
    return 0;
}

int grid_for_tiles(int64_t ntiles, int cap) {
    int64_t g = (ntiles + kWaves - 1) / kWaves;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (int)g;
}

// The reduce grid: every wave takes one run of R consecutive tiles and the
// hardware dispatcher issues the blocks in order, so the tiles in flight at
// any moment form one narrow window of each buffer.  (A persistent grid whose
// waves walk the shard measured 5-10% slower: its waves drift apart and the
// reads in flight spread over the buffers.  Tiles taken from a counter, as the
// update does, would make each block's partial sum depend on which tiles it
// took, and the norm on the run.)  A reduce of 16-bit or fp32
// inputs takes one tile per wave (R = 1): on 8 fp16 slices of 1.25e9 elements
// that measured 7-10% faster than runs of 16 tiles, whose waves work in as
// many separate windows.  It is issued as launches of at most kSliceBlocks
// blocks over consecutive tile ranges; with statistics every later launch
// adds its blocks' sums onto the partials the first one wrote.  R grows only
// when the shard would take more than kMaxLaunches launches.
// INT8 payloads and the statistics-only pass keep runs of about kRunSteps
// steps (a step is one tile of one buffer group; R shrinks so that small
// shards still launch kFillBlocks blocks and grows so that the blocks fit the
// partial sums): one launch, at 98% of the read-only rate for the latter.
constexpr int64_t kRunSteps = 16;
constexpr int64_t kFillBlocks = 4096;
constexpr int64_t kMaxLaunches = 64;
constexpr int64_t kMaxGridPlain = int64_t(1) << 30;   // no partial sums to hold
template <int DT, bool VEC, bool SHIFT, bool WRITE, bool STATS, int TU, int KC, bool ACC, bool G1>
bool launch_reduce_grid(const ReduceLaunch& a, void* stream, float inv_n, int pow2) {
    constexpr int64_t kT = 256 * TU;
    const int64_t hs = SHIFT ? a.head : 0;           // as the kernel splits the shard
    const int64_t nbody = a.n > hs ? a.n - hs : 0;
    const int64_t ntiles = (nbody + kT - 1) / kT;
    const int64_t nfull = VEC ? nbody / kT : 0;
    const int64_t ngroups = G1 ? 1 : a.n_ranks / KC;
    // reduces of 16-bit and fp32 inputs go in launch slices; INT8 payloads
    // and the statistics pass in one launch (fewer blocks than partials)
    const bool sliced = DT != kQ8 && WRITE;
    const int64_t cap = sliced ? kSliceBlocks : (STATS ? kMaxGridReduce : kMaxGridPlain);
    static_assert(kSliceBlocks <= kMaxGridReduce, "a launch slice holds one partial per block");
    // two blocks per compute unit for the shapes with TU x KC >= 16 quads
    // in flight per lane
    const bool two = WRITE && TU * KC >= 16;
    int64_t run;
    if (DT == kQ8 || !WRITE) {
        run = kRunSteps / ngroups;
        const int64_t fill = ntiles / (kWaves * kFillBlocks);
        if (run > fill) run = fill;
        if (run < 1) run = 1;
        const int64_t need = (ntiles + kWaves * cap - 1) / (kWaves * cap);
        if (run < need) run = need;
    } else {
        const int64_t span = kWaves * cap * kMaxLaunches;   // tiles at R = 1
        run = (nfull + span - 1) / span;
        if (run < 1) run = 1;
    }
    const int64_t per_block = kWaves * run;          // full tiles per block
    const int64_t chunk = cap * per_block;           // full tiles per launch
    int64_t t0 = 0;
    int part = kPartFirst;
    bool folded = false;
    for (;;) {
        const int64_t t1 = nfull - t0 > chunk ? t0 + chunk : nfull;
        const bool last = t1 == nfull;
        int64_t grid = (t1 - t0 + per_block - 1) / per_block;
        if (last) {   // the ragged tail's tiles go to the last launch's waves
            int64_t tail = (ntiles - nfull + kWaves - 1) / kWaves;
            if (tail > cap) tail = cap;
            if (grid < tail) grid = tail;
        }
        if (grid < 1) grid = 1;
        // a reduce of one small launch folds its own partial sums
        if (STATS && part == kPartFirst && last && grid <= kFoldThreads) {
            part |= kPartFold;
            folded = true;
        }
        const unsigned lds = two && grid >= kTwoBlocksMin ? kLdsTwoBlocks : 0u;
        hipLaunchKernelGGL((reduce_kernel<DT, VEC, SHIFT, WRITE, STATS, TU, KC, ACC, G1>),
                           dim3((unsigned)grid), dim3(kThreads), lds, (hipStream_t)stream, a, inv_n,
                           pow2, (int)run, t0, t1, part | (last ? kPartLast : 0));
        if (last) break;
        t0 = t1;
        part = kPartAdd;
    }
    return folded;
}

template <int DT, bool VEC, bool SHIFT, bool WRITE, bool STATS, int TU, int KC, bool ACC>
bool launch_reduce_shape(const ReduceLaunch& a, void* stream, float inv_n, int pow2) {
    if (a.n_ranks == KC)
        return launch_reduce_grid<DT, VEC, SHIFT, WRITE, STATS, TU, KC, ACC, true>(a, stream, inv_n, pow2);
    return launch_reduce_grid<DT, VEC, SHIFT, WRITE, STATS, TU, KC, ACC, false>(a, stream, inv_n, pow2);
}

template <int DT, bool VEC, bool SHIFT, bool WRITE, bool STATS, bool ACC>
int launch_reduce_t(const ReduceLaunch& a, void* stream) {
    const int N = a.n_ranks;
    const int pow2 = (N & (N - 1)) == 0;
    const float inv_n = 1.0f / (float)N;  // exact when N is a power of two
    // reads in flight per lane: TU chunks x KC buffers (KC divides N), and with
    // several buffer groups the next step's reads on top (the pipeline); a
    // wave takes one tile.  Measured with the statistics on 16-bit buffers
    // (TB/s, the kept shape first):
    //   64 buffers: 1 x 16 5.93, 2 x 16 5.67, 4 x 16 5.82 (1 x 16 was also 7%
    //               faster than 2 x 8 with runs of tiles)
    //   32: 2 x 16 6.07 against 1 x 16 5.73;  16: 2 x 16 6.01 against 1 x 16
    //   4.82 (one step: one chunk left too few reads in flight)
    //   8: 4 x 8 (a whole tile in one step) 4-8% faster than 2 x 8
    //   12: 4 x 4 6.15 against 2 x 4 5.81;  4: 2 x 4 6.18, 8 x 4 6.09, 4 x 4 5.45
    //   2 and 6: 4 x 2 6.25 / 6.10, 8 x 2 6.06 / 5.99
    //   odd (3): 4 x 1 6.22 against 8 x 1 5.87;  16 chunks per tile spill registers
    //   24 and 40 (several groups of 8): 1 x 8 5.79 / 6.04 against 2 x 8 5.70 / 5.84
    // fp32 buffers (two registers per value more): 2 x 8 for eight (6.08 against
    // 5.92 with 4 x 8), 4 x 4 for four (6.32 against 5.89 with 2 x 4), 4 x 1 for
    // three (6.08 against 5.62 with 8 x 1).  INT8 payloads: 2 x 8 (eight: 5.88
    // against 5.60 with 4 x 8 and 5.45 with 1 x 8; 64: within 2% of 4 x 8).
    constexpr bool k16 = DT == ZERO_F16 || DT == ZERO_BF16;
    constexpr int kTu16 = k16 ? 2 : 1;   // 16 or 32 16-bit buffers
    constexpr int kTu8 = k16 ? 1 : 2;    // 24, 40, 56, ... 16-bit buffers
    constexpr int kTu4 = k16 || DT == ZERO_F32 ? 4 : 2;
    constexpr int kTuOdd = DT == kQ8 ? 8 : 4;
    bool folded = false;
    if (DT != kQ8 && N % 16 == 0) {
        if (k16 && N <= 32)
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, kTu16, 16, ACC>(a, stream, inv_n, pow2);
        else
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, 1, 16, ACC>(a, stream, inv_n, pow2);
    } else if (k16 && N == 8) {
        folded = launch_reduce_grid<DT, VEC, SHIFT, WRITE, STATS, (k16 ? 4 : 2), 8, ACC, true>(
            a, stream, inv_n, pow2);
    } else if (N % 8 == 0) {
        if (k16)
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, kTu8, 8, ACC>(a, stream, inv_n, pow2);
        else
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, 2, 8, ACC>(a, stream, inv_n, pow2);
    } else if (N % 4 == 0) {
        if (k16 ? N > 4 : (DT == ZERO_F32 && N == 4))
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, kTu4, 4, ACC>(a, stream, inv_n, pow2);
        else
            folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, 2, 4, ACC>(a, stream, inv_n, pow2);
    } else if (N % 2 == 0) {
        folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, 4, 2, ACC>(a, stream, inv_n, pow2);
    } else if (N == 1) {
        folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, 2, 1, ACC>(a, stream, inv_n, pow2);
    } else {
        folded = launch_reduce_shape<DT, VEC, SHIFT, WRITE, STATS, kTuOdd, 1, ACC>(a, stream, inv_n, pow2);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    if (STATS && !folded) {
        hipLaunchKernelGGL(fold_kernel, dim3(1), dim3(kFoldThreads), 0, (hipStream_t)stream, a.st,
                           a.partials);
        e = hipGetLastError();
    }
    return (int)e;
}

template <int DT, bool VEC, bool SHIFT>
int launch_reduce_d(const ReduceLaunch& a, void* stream) {
    const bool write = a.red_out != nullptr;
    const bool stats = a.st != nullptr;
    if (write && a.accumulate) {
        if (stats) return launch_reduce_t<DT, VEC, SHIFT, true, true, true>(a, stream);
        return launch_reduce_t<DT, VEC, SHIFT, true, false, true>(a, stream);
    }
    if (write && stats) return launch_reduce_t<DT, VEC, SHIFT, true, true, false>(a, stream);
    if (write) return launch_reduce_t<DT, VEC, SHIFT, true, false, false>(a, stream);
    return launch_reduce_t<DT, VEC, SHIFT, false, true, false>(a, stream);
}

template <int DT>
int launch_reduce_v(const ReduceLaunch& a, void* stream) {
    if (!a.vec) return launch_reduce_d<DT, false, false>(a, stream);
    return a.head ? launch_reduce_d<DT, true, true>(a, stream) : launch_reduce_d<DT, true, false>(a, stream);
}

// quantised payload: always writes the fp32 shard; statistics optional
template <bool VEC>
int launch_reduce_q8_v(const ReduceLaunch& a, void* stream) {
    if (a.st) return launch_reduce_t<kQ8, VEC, false, true, true, false>(a, stream);
    return launch_reduce_t<kQ8, VEC, false, true, false, false>(a, stream);
}

template <int GT, int PT, bool QUANT>
int launch_adamw_q(const AdamLaunch& a, void* stream) {
    const int64_t ntiles = (a.n + kTile - 1) / kTile;
    const int64_t ngroups = (ntiles + kWaves - 1) / kWaves;
    if (a.vec && ngroups >= kSchedMinGroups) {
        int cus = 0;
        const int e = cu_count_for_current_device(&cus);
        if (e) return e;
        int64_t grid = 2 * (int64_t)cus;                // two blocks per compute unit
        if (grid > ngroups) grid = ngroups;
        hipLaunchKernelGGL((adamw_sched_kernel<GT, PT, QUANT>), dim3((unsigned)grid),
                           dim3(kThreads), kLdsTwoBlocks, (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const int64_t slice = kSliceBlocks * kWaves;   // tiles per launch
    for (int64_t t0 = 0; t0 < ntiles; t0 += slice) {
        const int64_t t1 = ntiles - t0 < slice ? ntiles : t0 + slice;
        const int grid = grid_for_tiles(t1 - t0, kMaxGridStep);
        const unsigned lds = !QUANT && grid >= kTwoBlocksMin ? kLdsTwoBlocks : 0u;
        if (a.vec)
            hipLaunchKernelGGL((adamw_kernel<GT, PT, QUANT, true>), dim3(grid), dim3(kThreads),
                               lds, (hipStream_t)stream, a, t0, t1);
        else
            hipLaunchKernelGGL((adamw_kernel<GT, PT, QUANT, false>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a, t0, t1);
    }
    return (int)hipGetLastError();
}

template <int GT, int PT>
int launch_adamw_p(const AdamLaunch& a, void* stream) {
    return a.q ? launch_adamw_q<GT, PT, true>(a, stream) : launch_adamw_q<GT, PT, false>(a, stream);
}

template <int GT>
int launch_adamw_g(const AdamLaunch& a, void* stream) {
    return a.pdtype == ZERO_F16 ? launch_adamw_p<GT, ZERO_F16>(a, stream)
                                : launch_adamw_p<GT, ZERO_BF16>(a, stream);
}

}  // namespace

int launch_reduce_q8(const ReduceLaunch& a, void* stream) {
    return a.vec ? launch_reduce_q8_v<true>(a, stream) : launch_reduce_q8_v<false>(a, stream);
}

int launch_reduce_stats(const ReduceLaunch& a, void* stream) {
    switch (a.dtype) {
        case ZERO_F32: return launch_reduce_v<ZERO_F32>(a, stream);
        case ZERO_F16: return launch_reduce_v<ZERO_F16>(a, stream);
        default: return launch_reduce_v<ZERO_BF16>(a, stream);
    }
}

}  // namespace zf

// ---------------------------------------------------------------- library-owned scratch
// The statistics' per-block partial sums for zero_grad_reduce_shard_noalloc,
// for callers that cannot allocate: one array per device, held until the
// process ends.  Every such call on a device shares it (calls that overlap on
// one device race); the first launch of a reduce writes every partial its fold
// reads (later launches of the same reduce add onto them), so nothing needs
// clearing between calls.
static __device__ __align__(256) double scratch[ZERO_MAX_PARTIALS];

namespace zf {
namespace {
// scratch's device address on each device, looked up once per device (with
// that device current) on the first no-allocation call there.  In host code
// the array's name is only a stand-in for the symbol; kernels get this
// address instead.
constexpr int kMaxDevices = 64;
std::atomic<double*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_current_device(double** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    double* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return (int)e;
            if (!addr) return (int)hipErrorInvalidSymbol;
            p = static_cast<double*>(addr);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return 0;
}
}  // namespace

int launch_reduce_noalloc(ReduceLaunch& a, void* stream) {
    if (a.st) {
        // the grid never exceeds ZERO_MAX_PARTIALS blocks (runs lengthen
        // instead), which is what the scratch holds
        static_assert(kMaxGridReduce <= ZERO_MAX_PARTIALS, "scratch smaller than the grid cap");
        int e = scratch_for_current_device(&a.partials);
        if (e) return e;
    }
    return launch_reduce_stats(a, stream);
}

int launch_adamw(const AdamLaunch& a, void* stream) {
    if (a.n > 0) {
        int e;
        switch (a.gdtype) {
            case ZERO_F32: e = launch_adamw_g<ZERO_F32>(a, stream); break;
            case ZERO_F16: e = launch_adamw_g<ZERO_F16>(a, stream); break;
            default: e = launch_adamw_g<ZERO_BF16>(a, stream); break;
        }
        if (e != 0) return e;
    }
    if (a.flags & ZERO_STEP_FINALIZE) {
        hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, a.st,
                           a.beta1, a.beta2, a.max_norm);
        return (int)hipGetLastError();
    }
    return 0;
}

int launch_dequant(const DequantLaunch& a, void* stream) {
    const int64_t per_slot = (a.slot_numel + kDTile - 1) / kDTile;
    const bool flat = a.vec && a.slot_numel >= kDTile;
    const int64_t ntiles = flat ? (a.slot_numel * a.n_slots + kDTile - 1) / kDTile
                                : per_slot * a.n_slots;
    const int grid = grid_for_tiles(ntiles, kMaxGridStream);
    const int64_t slice = kSliceBlocks * kWaves;   // flat tiles per launch
    int shift = -1;
    if ((a.block & (a.block - 1)) == 0) shift = __builtin_ctz((unsigned)a.block);
    hipStream_t s = (hipStream_t)stream;
#define ZF_DQ(OT)                                                                           \
    do {                                                                                    \
        if (flat) {                                                                         \
            for (int64_t t0 = 0; t0 < ntiles; t0 += slice) {                                \
                const int64_t t1 = ntiles - t0 < slice ? ntiles : t0 + slice;              \
                hipLaunchKernelGGL((dequant_flat_kernel<OT>),                                \
                                   dim3(grid_for_tiles(t1 - t0, kMaxGridStream)), dim3(kThreads), \
                                   0, s, a, shift, t0, t1);                                 \
            }                                                                               \
        } else if (a.vec) hipLaunchKernelGGL((dequant_kernel<OT, true>), dim3(grid), dim3(kThreads), 0, s, a, shift); \
        else hipLaunchKernelGGL((dequant_kernel<OT, false>), dim3(grid), dim3(kThreads), 0, s, a, shift);      \
    } while (0)
    if (a.out_dtype == ZERO_F32) ZF_DQ(ZERO_F32);
    else if (a.out_dtype == ZERO_F16) ZF_DQ(ZERO_F16);
    else ZF_DQ(ZERO_BF16);
#undef ZF_DQ
    return (int)hipGetLastError();
}

int launch_quant(const QuantLaunch& a, void* stream) {
    if (a.vec == 2) {
        const int grid = grid_for_tiles((a.n + kQTile - 1) / kQTile, kMaxGridStream);
        if (a.dtype == ZERO_F16)
            hipLaunchKernelGGL((quant8_kernel<ZERO_F16>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
        else
            hipLaunchKernelGGL((quant8_kernel<ZERO_BF16>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const int64_t ntiles = (a.n + kTile - 1) / kTile;
    const int grid = grid_for_tiles(ntiles, kMaxGridStep);
    if (a.dtype == ZERO_F16) {
        if (a.vec)
            hipLaunchKernelGGL((quant_kernel<ZERO_F16, true>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
        else
            hipLaunchKernelGGL((quant_kernel<ZERO_F16, false>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
    } else {
        if (a.vec)
            hipLaunchKernelGGL((quant_kernel<ZERO_BF16, true>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
        else
            hipLaunchKernelGGL((quant_kernel<ZERO_BF16, false>), dim3(grid), dim3(kThreads), 0,
                               (hipStream_t)stream, a);
    }
    return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace zf
