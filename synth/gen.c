/*
 * Counter-based seeded input generator (host side).
 *
 * This module only draws synthetic inputs (weights, caches, token ids). It
 * holds none of the Dual-Flow arithmetic. Both the CPU oracle and the GPU
 * path take their inputs from here (the GPU twin in gen_dev.hip computes the
 * same function bit for bit).
 *
 * Definition (every value is a pure function of (seed, stream, index)):
 *   mix64(z)  : the SplitMix64 output finaliser of Steele, Lea and Flood,
 *               "Fast splittable pseudorandom number generators" (OOPSLA 2014):
 *               z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *               z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key(s,t)  = mix64(mix64(s + G) ^ t), G = 0x9E3779B97F4A7C15 (golden gamma)
 *   word(k,i) = mix64(k + (i+1)*G)     -- SplitMix64 state k advanced i+1 times
 *   normal    : Irwin-Hall sum of the four 16-bit fields of word, centred and
 *               scaled to unit variance, n = sum - 131070 (exact integer),
 *               value = (float)((double)n * (sigma / sqrt((65536^2-1)/3)))
 *               (one double multiply, one round to fp32: IEEE, portable).
 *   bf16      : fp32 -> bf16 round-to-nearest-even on the bit pattern.
 *   uniform   : lo + ((word >> 32) * (hi - lo)) >> 32, in [lo, hi).
 */
#include <stdint.h>
#include <math.h>
#include <string.h>

#define G64 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed + G64) ^ stream);
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * G64);
}

/* Scale that maps the centred 4x16-bit sum to unit variance. */
static double inv_std(void) { return 1.0 / sqrt((65536.0 * 65536.0 - 1.0) / 3.0); }

static inline float normal_at(uint64_t key, uint64_t i, double scale) {
    uint64_t w = word_at(key, i);
    int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
                (int32_t)((w >> 32) & 0xFFFF) + (int32_t)(w >> 48);
    int32_t n = s - 131070;
    return (float)((double)n * scale);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) {           /* inf / nan */
        return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_words(uint64_t* out, int64_t n, uint64_t key, int64_t offset) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = word_at(key, (uint64_t)(offset + i));
}

void synth_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream,
                      int64_t offset, double sigma) {
    uint64_t key = synth_key(seed, stream);
    double scale = sigma * inv_std();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, (uint64_t)(offset + i), scale);
}

void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream,
                       int64_t offset, double sigma) {
    uint64_t key = synth_key(seed, stream);
    double scale = sigma * inv_std();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(normal_at(key, (uint64_t)(offset + i), scale));
}

/* Many streams at once: stream s of n_per elements goes to out + s*pitch.
 * Stream ids are stream0 + s*stream_step. Used for per-(layer, seq, head)
 * cache blocks. */
void synth_normal_bf16_streams(uint16_t* out, int64_t n_streams, int64_t n_per,
                               int64_t pitch, uint64_t seed, const uint64_t* streams,
                               double sigma) {
    double scale = sigma * inv_std();
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n_streams; ++s) {
        uint64_t key = synth_key(seed, streams[s]);
        uint16_t* o = out + s * pitch;
        for (int64_t i = 0; i < n_per; ++i) o[i] = f32_to_bf16_rne(normal_at(key, (uint64_t)i, scale));
    }
}

void synth_normal_f32_streams(float* out, int64_t n_streams, int64_t n_per,
                              int64_t pitch, uint64_t seed, const uint64_t* streams,
                              double sigma) {
    double scale = sigma * inv_std();
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n_streams; ++s) {
        uint64_t key = synth_key(seed, streams[s]);
        float* o = out + s * pitch;
        for (int64_t i = 0; i < n_per; ++i) o[i] = normal_at(key, (uint64_t)i, scale);
    }
}

void synth_uniform_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t stream,
                       int64_t offset, int32_t lo, int32_t hi) {
    uint64_t key = synth_key(seed, stream);
    uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t w = word_at(key, (uint64_t)(offset + i));
        out[i] = lo + (int32_t)(((w >> 32) * span) >> 32);
    }
}
