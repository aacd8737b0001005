/*
 * synth_gpu.hip -- seeded synthetic inputs on the GPU, plus the streaming
 * calibration kernels (copy, read-only, write-only, and the byte mix of a
 * fused AdamW update with trivial arithmetic) that measure the practical HBM
 * ceilings beside the step and calibrate the traffic counters.  Holds none of
 * the optimizer step's arithmetic.
 *
 * The generator is the same definition as synth_cpu.c, implemented
 * independently here:
 *   SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output n of the stream
 *   seeded with `key` is mix(key + (n+1)*0x9e3779b97f4a7c15), mix being
 *   z ^= z>>30; z *= 0xbf58476d1ce4e5b9; z ^= z>>27; z *= 0x94d049bb133111eb;
 *   z ^= z>>31.  Element j sums the twelve 16-bit fields of outputs 3j..3j+2
 *   (Irwin-Hall(12)): z = (2*sum - 786420) * 2^-17, exact in integers and
 *   exactly representable in binary32; value = z * sigma (one rounding),
 *   then rounded to nearest-even into the storage format (on the bits).
 *   Integer codes in [-127, 127]: element j takes output j, hi = its high 32
 *   bits, code = floor(hi * 255 / 2^32) - 127.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float unit_variate(uint64_t key, uint64_t j) {
    int64_t s = 0;
#pragma unroll
    for (uint64_t r = 0; r < 3; ++r) {
        const uint64_t h = mix64(key + (3u * j + r + 1u) * kGamma);
        s += (int64_t)(h & 0xffffu) + (int64_t)((h >> 16) & 0xffffu) +
             (int64_t)((h >> 32) & 0xffffu) + (int64_t)(h >> 48);
    }
    const int32_t zi = (int32_t)(2 * s - 12 * 65535);
    return (float)zi * 0x1p-17f;
}

/* Round-to-nearest-even of binary32 to the storage format, on the bit
 * patterns (no hardware conversion mode involved). */
__device__ __forceinline__ uint16_t to_half_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t h;
    if (a >= 0x7f800000u) h = a > 0x7f800000u ? 0x7e00u : 0x7c00u;
    else if (a >= 0x477ff000u) h = 0x7c00u;
    else if (a >= 0x38800000u) { const uint32_t m = a - 0x38000000u; h = (m + 0xfffu + ((m >> 13) & 1u)) >> 13; }
    else h = __float_as_uint(__uint_as_float(a) + 0.5f) - 0x3f000000u;
    return (uint16_t)(sign | h);
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int DT, typename T>
__global__ void __launch_bounds__(256) fill_normal(uint64_t key, int64_t start, int64_t n,
                                                   float sigma, T* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = unit_variate(key, (uint64_t)(start + i)) * sigma;
        if constexpr (DT == 0) out[i] = x;
        else if constexpr (DT == 1) out[i] = to_half_bits(x);
        else out[i] = to_bf16_bits(x);
    }
}

__global__ void __launch_bounds__(256) fill_codes(uint64_t key, int64_t start, int64_t n,
                                                  int8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint64_t hi = mix64(key + ((uint64_t)(start + i) + 1u) * kGamma) >> 32;
        out[i] = (int8_t)((int64_t)((hi * 255u) >> 32) - 127);
    }
}

/* Plain streaming copy of 16-byte words: the reference kernel whose
 * FETCH_SIZE/WRITE_SIZE per byte calibrate the counters and whose time is
 * the practical read+write ceiling.  A block copies one contiguous span of
 * 1024 words (16 KiB): each thread loads four words 256 apart, then stores
 * them, with non-temporal accesses (every byte is touched once), and blocks
 * loop over spans when the grid is smaller than the copy. */
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__global__ void __launch_bounds__(256) copy16(const u32x4* __restrict__ src,
                                              u32x4* __restrict__ dst, int64_t n16) {
    for (int64_t b = (int64_t)blockIdx.x * 1024; b < n16; b += (int64_t)gridDim.x * 1024) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = b + 256 * k + threadIdx.x;
            if (i < n16) v[k] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = b + 256 * k + threadIdx.x;
            if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
        }
    }
}

/* Read-only stream of 16-byte words (non-temporal), 16 KiB per block and
 * pass; the XOR of the words is stored only if it equals `never`, which keeps
 * the loads live. */
__global__ void __launch_bounds__(256) read16(const u32x4* __restrict__ src, int64_t n16,
                                              uint32_t never, uint32_t* __restrict__ sink) {
    uint32_t x = 0;
    for (int64_t b = (int64_t)blockIdx.x * 1024; b < n16; b += (int64_t)gridDim.x * 1024) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = b + 256 * k + threadIdx.x;
            v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4)(0u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (x == never) sink[0] = x;
}

/* Read-only pass over up to kMaxStreams buffers of the same size at once: a
 * block reads 256 consecutive 8-byte words of every buffer (one per thread),
 * 16 buffers in flight; the sum is stored only if it equals `never`, which
 * keeps the loads live. */
constexpr int kMaxStreams = 128;
struct StreamPtrs {
    const u32x2* p[kMaxStreams];
};
template <int KC>
__global__ void __launch_bounds__(256) read_streams8(StreamPtrs b, int nbuf, int64_t w0,
                                                     int64_t nw, uint32_t never,
                                                     uint32_t* __restrict__ sink) {
    const int64_t i = w0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    if (i < nw) {
        for (int k0 = 0; k0 < nbuf; k0 += KC) {
            u32x2 v[KC];
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) v[kk] = __builtin_nontemporal_load(b.p[k0 + kk] + i);
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) x += v[kk].x ^ v[kk].y;
        }
    }
    if (x == never) sink[0] = x;
}

/* Write-only stream of 16-byte words (non-temporal), 16 KiB per block and pass. */
__global__ void __launch_bounds__(256) write16(u32x4* __restrict__ dst, int64_t n16, uint32_t val) {
    for (int64_t b = (int64_t)blockIdx.x * 1024; b < n16; b += (int64_t)gridDim.x * 1024) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = b + 256 * k + threadIdx.x;
            if (i < n16) __builtin_nontemporal_store((u32x4)(val), dst + i);
        }
    }
}

/* The byte mix of the fused update with trivial arithmetic: per element a
 * 16-bit g and fp32 p, m, v are read, p, m, v and a 16-bit copy of p are
 * written (14 B in, 14 B out), in the update's layout (one 1024-element tile
 * per wave; in slice u lane l holds elements 256u + 4l .. 4l+3) with
 * non-temporal accesses.  ntiles full tiles, one per wave. */
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) mix28(const uint16_t* __restrict__ g, float* __restrict__ p,
                                             float* __restrict__ m, float* __restrict__ v,
                                             uint16_t* __restrict__ lp, int64_t ntiles) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntiles) return;
    u32x2 gw[4];
    f32x4 pv[4], mv[4], vv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i0 = t * 1024 + 256 * u + 4 * lane;
        gw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(g + i0));
        pv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i0));
        mv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m + i0));
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v + i0));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i0 = t * 1024 + 256 * u + 4 * lane;
        const float gf = (float)(gw[u].x & 0xffffu);
        f32x4 a = pv[u], b = mv[u], c = vv[u];
        a.x = a.x + gf; b.x = b.x + gf; c.x = c.x + gf;
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p + i0));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(m + i0));
        __builtin_nontemporal_store(c, reinterpret_cast<f32x4*>(v + i0));
        u32x2 o;
        o.x = (__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xffff0000u);
        o.y = (__float_as_uint(a.z) >> 16) | (__float_as_uint(a.w) & 0xffff0000u);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(lp + i0));
    }
}

int grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

extern "C" {

/* dtype: 0 = fp32, 1 = fp16, 2 = bf16.  Returns 0 or a hipError_t. */
int synth_fill_normal(uint64_t key, int64_t start, int64_t n, float sigma, void* out,
                      int32_t dtype, void* stream) {
    if (n <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    const int g = grid_for(n);
    if (dtype == 0)
        hipLaunchKernelGGL((fill_normal<0, float>), dim3(g), dim3(256), 0, s, key, start, n,
                           sigma, (float*)out);
    else if (dtype == 1)
        hipLaunchKernelGGL((fill_normal<1, uint16_t>), dim3(g), dim3(256), 0, s, key, start, n,
                           sigma, (uint16_t*)out);
    else if (dtype == 2)
        hipLaunchKernelGGL((fill_normal<2, uint16_t>), dim3(g), dim3(256), 0, s, key, start, n,
                           sigma, (uint16_t*)out);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

/* nbytes must be a multiple of 16 and both pointers 16-byte aligned. */
/* out[i] = integer code of (key, start + i) in [-127, 127]. */
int synth_fill_codes(uint64_t key, int64_t start, int64_t n, int8_t* out, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(fill_codes, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key,
                       start, n, out);
    return (int)hipGetLastError();
}

/* Launch form of the calibration streams below (copy without an explicit
 * grid, read, write, mix28): 0 = one launch; else consecutive launches of at
 * most slice_blocks blocks over consecutive spans (tiles), each with lds_bytes
 * of dynamic LDS reserved (unused; it caps the blocks resident per compute
 * unit).  The same forms as the library's streaming kernels, so that their
 * ceilings are measured in the launch form the kernels use. */
static int64_t g_slice_blocks = 0;
static unsigned g_lds_bytes = 0;

int synth_set_launch_form(int64_t slice_blocks, uint32_t lds_bytes) {
    if (slice_blocks < 0 || lds_bytes > 80u * 1024u) return (int)hipErrorInvalidValue;
    g_slice_blocks = slice_blocks;
    g_lds_bytes = lds_bytes;
    return 0;
}

// spans of 1024 16-byte words per launch (all of them in one launch by default)
// (at most 2^22 blocks of 256 threads per launch: HIP's 2^32-thread grid limit)
static int64_t spans_per_launch(int64_t spans) {
    int64_t per = g_slice_blocks > 0 && g_slice_blocks < spans ? g_slice_blocks : spans;
    return per > (1 << 22) ? (1 << 22) : per;
}

int synth_copy(const void* src, void* dst, int64_t nbytes, int32_t grid, void* stream) {
    if (nbytes <= 0) return 0;
    if ((nbytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return (int)hipErrorInvalidValue;
    const int64_t n16 = nbytes / 16;
    int64_t spans = (n16 + 1023) / 1024;
    if (grid > 0 || spans > (1 << 22)) {   // one launch, blocks looping over spans
        if (spans > (1 << 22)) spans = 1 << 22;
        const int g = grid > 0 ? grid : (int)spans;
        hipLaunchKernelGGL(copy16, dim3(g), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                           (u32x4*)dst, n16);
        return (int)hipGetLastError();
    }
    const int64_t per = spans_per_launch(spans);
    for (int64_t s0 = 0; s0 < spans; s0 += per) {
        const int64_t w0 = s0 * 1024;
        const int64_t nw = n16 - w0 < per * 1024 ? n16 - w0 : per * 1024;
        hipLaunchKernelGGL(copy16, dim3((int)((nw + 1023) / 1024)), dim3(256), g_lds_bytes,
                           (hipStream_t)stream, (const u32x4*)src + w0, (u32x4*)dst + w0, nw);
    }
    return (int)hipGetLastError();
}

/* Read-only stream over nbytes (a multiple of 16, 16-byte aligned); sink:
 * one writable uint32. */
int synth_read(const void* src, int64_t nbytes, void* sink, void* stream) {
    if (nbytes <= 0) return 0;
    if ((nbytes & 15) || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
    const int64_t n16 = nbytes / 16;
    const int64_t spans = (n16 + 1023) / 1024;
    const int64_t per = spans_per_launch(spans);
    for (int64_t s0 = 0; s0 < spans; s0 += per) {
        const int64_t w0 = s0 * 1024;
        const int64_t nw = n16 - w0 < per * 1024 ? n16 - w0 : per * 1024;
        hipLaunchKernelGGL(read16, dim3((int)((nw + 1023) / 1024)), dim3(256), g_lds_bytes,
                           (hipStream_t)stream, (const u32x4*)src + w0, nw, 0x9e3779b9u,
                           (uint32_t*)sink);
    }
    return (int)hipGetLastError();
}

/* Read-only pass over nbuf buffers of nbytes each at once (bufs: a host
 * array of device pointers; nbytes a multiple of 8, every buffer 8-byte
 * aligned; 1 <= nbuf <= 128); sink: one writable uint32. */
int synth_read_streams(const void* const* bufs, int32_t nbuf, int64_t nbytes, void* sink,
                       void* stream) {
    if (nbytes <= 0) return 0;
    if (nbuf < 1 || nbuf > kMaxStreams || (nbytes & 7)) return (int)hipErrorInvalidValue;
    StreamPtrs b;
    for (int k = 0; k < kMaxStreams; ++k) b.p[k] = nullptr;
    for (int k = 0; k < nbuf; ++k) {
        if (!bufs[k] || ((uintptr_t)bufs[k] & 7)) return (int)hipErrorInvalidValue;
        b.p[k] = (const u32x2*)bufs[k];
    }
    const int64_t nw = nbytes / 8;
    const int64_t blocks = (nw + 255) / 256;
    const int64_t per = spans_per_launch(blocks);
    for (int64_t s0 = 0; s0 < blocks; s0 += per) {
        const int64_t nb = blocks - s0 < per ? blocks - s0 : per;
        const int64_t w0 = s0 * 256;
        if (nbuf % 16 == 0)
            hipLaunchKernelGGL(read_streams8<16>, dim3((unsigned)nb), dim3(256), g_lds_bytes,
                               (hipStream_t)stream, b, nbuf, w0, nw, 0x9e3779b9u, (uint32_t*)sink);
        else if (nbuf % 8 == 0)
            hipLaunchKernelGGL(read_streams8<8>, dim3((unsigned)nb), dim3(256), g_lds_bytes,
                               (hipStream_t)stream, b, nbuf, w0, nw, 0x9e3779b9u, (uint32_t*)sink);
        else
            hipLaunchKernelGGL(read_streams8<1>, dim3((unsigned)nb), dim3(256), g_lds_bytes,
                               (hipStream_t)stream, b, nbuf, w0, nw, 0x9e3779b9u, (uint32_t*)sink);
    }
    return (int)hipGetLastError();
}

/* Write-only stream over nbytes (a multiple of 16, 16-byte aligned). */
int synth_write(void* dst, int64_t nbytes, uint32_t val, void* stream) {
    if (nbytes <= 0) return 0;
    if ((nbytes & 15) || ((uintptr_t)dst & 15)) return (int)hipErrorInvalidValue;
    const int64_t n16 = nbytes / 16;
    const int64_t spans = (n16 + 1023) / 1024;
    const int64_t per = spans_per_launch(spans);
    for (int64_t s0 = 0; s0 < spans; s0 += per) {
        const int64_t w0 = s0 * 1024;
        const int64_t nw = n16 - w0 < per * 1024 ? n16 - w0 : per * 1024;
        hipLaunchKernelGGL(write16, dim3((int)((nw + 1023) / 1024)), dim3(256), g_lds_bytes,
                           (hipStream_t)stream, (u32x4*)dst + w0, nw, val);
    }
    return (int)hipGetLastError();
}

/* The fused update's byte mix over n elements (n a multiple of 1024; p, m, v
 * 16-byte and g, lp 8-byte aligned). */
int synth_mix28(const void* g, float* p, float* m, float* v, void* lp, int64_t n, void* stream) {
    if (n <= 0) return 0;
    if ((n & 1023) || ((uintptr_t)g & 7) || ((uintptr_t)lp & 7) || ((uintptr_t)p & 15) ||
        ((uintptr_t)m & 15) || ((uintptr_t)v & 15))
        return (int)hipErrorInvalidValue;
    const int64_t ntiles = n / 1024;
    const int64_t blocks = (ntiles + 3) / 4;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    const int64_t per = 4 * spans_per_launch(blocks);   // tiles per launch
    for (int64_t t0 = 0; t0 < ntiles; t0 += per) {
        const int64_t nt = ntiles - t0 < per ? ntiles - t0 : per;
        const int64_t e0 = t0 * 1024;
        hipLaunchKernelGGL(mix28, dim3((unsigned)((nt + 3) / 4)), dim3(256), g_lds_bytes,
                           (hipStream_t)stream, (const uint16_t*)g + e0, p + e0, m + e0, v + e0,
                           (uint16_t*)lp + e0, nt);
    }
    return (int)hipGetLastError();
}

}  // extern "C"
