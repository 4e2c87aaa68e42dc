/*
 * Seeded synthetic-input generator shared by the oracle tests and the HIP
 * path. It holds none of the MoE layer's arithmetic: it only turns
 * (seed, tag, element index) into normally distributed values rounded to
 * bfloat16, so any slice of any tensor can be regenerated independently and
 * both sides consume identical bits.
 *
 * Counter-based generator: each 64-bit draw is the SplitMix64 output
 * function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) applied to  key + (counter + 1) * golden-gamma,
 * where key = mix(seed ^ mix(tag)). Two draws per element feed the
 * Box-Muller transform in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t GOLDEN_GAMMA = 0x9E3779B97F4A7C15ULL;

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t tag) {
    return mix64(seed ^ mix64(tag + GOLDEN_GAMMA));
}

static uint64_t draw(uint64_t key, uint64_t counter) {
    return mix64(key + (counter + 1) * GOLDEN_GAMMA);
}

/* Standard normal for element i of stream (seed, tag). */
static double normal_at(uint64_t key, uint64_t i) {
    uint64_t a = draw(key, 2 * i), b = draw(key, 2 * i + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* double -> float (round to nearest even by the C conversion) -> bf16 bits
 * (round to nearest even on the dropped 16 bits). Inputs are finite. */
static uint16_t to_bf16_bits(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[j] = bf16(std * N(0,1) at element start + j) for j < n. */
void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t start, uint64_t n, double std,
                       uint16_t* out) {
    uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = to_bf16_bits(std * normal_at(key, start + (uint64_t)j));
}

/* Same stream in double precision, unrounded (used for biases). */
void synth_normal_f64(uint64_t seed, uint64_t tag, uint64_t start, uint64_t n, double std, double* out) {
    uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = std * normal_at(key, start + (uint64_t)j);
}

/* Raw 64-bit draws (used for seeded permutations). */
void synth_u64(uint64_t seed, uint64_t tag, uint64_t start, uint64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, tag);
    for (uint64_t j = 0; j < n; ++j) out[j] = draw(key, start + j);
}
