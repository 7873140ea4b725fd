/*
 * Seeded synthetic inputs for the gated temporal scan.
 *
 * A counter-based normal generator: element n of tensor `tid` under `seed`
 * depends only on (seed, tid, n), so the result is independent of thread
 * count and of how the array is split.
 *
 *   SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): state advances by the golden-ratio increment
 *   0x9E3779B97F4A7C15 and each output is the 64-bit finaliser applied to
 *   the new state.  Output n of a stream started at state s0 is therefore
 *   mix(s0 + (n + 1) * increment).
 *
 *   Stream key: s0 = mix(seed * 256 + tid + increment), i.e. the first
 *   SplitMix64 output of a generator seeded with (seed << 8 | tid).
 *
 *   Element n draws two outputs of that stream, z1 = out(2n), z2 = out(2n+1),
 *   turns them into u1 in (0, 1] and u2 in [0, 1) from their top 53 bits, and
 *   applies the Box-Muller transform (Box & Muller, Ann. Math. Stat. 1958):
 *   N = sqrt(-2 ln u1) * cos(2 pi u2), in double precision.  The value is
 *   scaled by `stddev` in double and rounded once to float (round to nearest
 *   even).
 *
 * This file holds no part of the scan itself; both the HIP path and the CPU
 * oracle receive the arrays it writes.
 */
#include <math.h>
#include <stdint.h>

#define SM64_INC 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* First output of a SplitMix64 generator whose state is `state`. */
uint64_t gscan_synth_splitmix64_first(uint64_t state)
{
    return sm64_mix(state + SM64_INC);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t tid)
{
    return gscan_synth_splitmix64_first(seed * 256ULL + (uint64_t)tid);
}

/* Output number `n` (0-based) of the stream that starts at state `key`. */
static inline uint64_t stream_out(uint64_t key, uint64_t n)
{
    return sm64_mix(key + (n + 1ULL) * SM64_INC);
}

double gscan_synth_normal_one(uint64_t seed, uint32_t tid, int64_t n)
{
    const uint64_t key = stream_key(seed, tid);
    const uint64_t z1 = stream_out(key, 2ULL * (uint64_t)n);
    const uint64_t z2 = stream_out(key, 2ULL * (uint64_t)n + 1ULL);
    const double u1 = ((double)(z1 >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    const double u2 = (double)(z2 >> 11) * 0x1.0p-53;         /* [0, 1) */
    const double two_pi = 6.283185307179586476925286766559;
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* out[i] = (float)(stddev * N(seed, tid, first + i)) for i in [0, count). */
void gscan_synth_normal_f32(uint64_t seed, uint32_t tid, double stddev,
                            int64_t first, int64_t count, float *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        out[i] = (float)(stddev * gscan_synth_normal_one(seed, tid, first + i));
}

/* Round float32 to bfloat16, nearest-even, returned as the raw 16 bits.
 * Inputs here are finite (normal draws), so no NaN handling is needed. */
void gscan_synth_round_bf16(const float *in, int64_t count, uint16_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        union { float f; uint32_t u; } v;
        v.f = in[i];
        const uint32_t lsb = (v.u >> 16) & 1u;
        out[i] = (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
    }
}
