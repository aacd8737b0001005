/*
 * synth_cpu.c -- seeded synthetic inputs on the host (CPU side).
 *
 * Holds none of the optimizer step's arithmetic.  The same generator is
 * implemented independently for the GPU in synth_gpu.hip; a GPU test checks
 * that both give identical bits.
 *
 * Generator (counter-based, random access by element index):
 *   SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number
 *   Generators", OOPSLA 2014; the output mixer with constants
 *   0xbf58476d1ce4e5b9 / 0x94d049bb133111eb and increment
 *   0x9e3779b97f4a7c15 as in Java's SplittableRandom): the n-th output of
 *   the stream seeded with `key` is mix(key + (n+1)*gamma).
 *   Element j uses outputs 3j, 3j+1, 3j+2; their twelve 16-bit fields
 *   u_0..u_11 form the Irwin-Hall(12) variate
 *       z = (2*sum(u) - 12*65535) * 2^-17      (mean 0, variance ~1, |z| <= 6)
 *   computed exactly in integers, converted exactly to binary32; the value
 *   is z * sigma rounded once to binary32.
 *
 * Integer codes in [-127, 127] (stand-ins for a gathered INT8 payload):
 *   element j uses output j alone, h = mix(key + (j+1)*gamma); its high 32
 *   bits hi give code = floor(hi * 255 / 2^32) - 127.
 */
#include <stdint.h>

static const uint64_t GAMMA = 0x9e3779b97f4a7c15ull;

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static float unit_variate(uint64_t key, uint64_t j) {
    int64_t s = 0;
    for (uint64_t r = 0; r < 3; ++r) {
        const uint64_t h = mix64(key + (3u * j + r + 1u) * GAMMA);
        s += (int64_t)(h & 0xffffu) + (int64_t)((h >> 16) & 0xffffu) +
             (int64_t)((h >> 32) & 0xffffu) + (int64_t)(h >> 48);
    }
    const int64_t zi = 2 * s - 12 * 65535;
    return (float)zi * 0x1p-17f;
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

/* out[i] = sigma * z(key, start + i), i in [0, n) */
void synth_normal_f32(uint64_t key, int64_t start, int64_t n, float sigma, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = unit_variate(key, (uint64_t)(start + i)) * sigma;
}

/* out[i] = sigma * z(key, idx[i]) */
void synth_normal_f32_at(uint64_t key, const int64_t* idx, int64_t n, float sigma, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = unit_variate(key, (uint64_t)idx[i]) * sigma;
}

static int8_t code_of(uint64_t key, uint64_t j) {
    const uint64_t hi = mix64(key + (j + 1u) * GAMMA) >> 32;
    return (int8_t)((int64_t)((hi * 255u) >> 32) - 127);
}

/* out[i] = code(key, start + i), i in [0, n) */
void synth_codes_i8(uint64_t key, int64_t start, int64_t n, int8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = code_of(key, (uint64_t)(start + i));
}

/* out[i] = code(key, idx[i]) */
void synth_codes_i8_at(uint64_t key, const int64_t* idx, int64_t n, int8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = code_of(key, (uint64_t)idx[i]);
}
