/*
 * Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.
 *
 * This file holds no arithmetic of the decode method: only a counter-based
 * random stream and table lookups. Every draw is a SplitMix64 output
 * (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), addressed by (seed, tensor id, element index) so that any
 * element of a 30-billion-element weight set can be produced independently,
 * in parallel, and identically on every machine.
 *
 *   normal fp16 : out[i] = table[draw >> 48], where the 65536-entry table holds
 *                 fp16 values of mu + sigma * Phi^-1((j + 0.5) / 65536)
 *                 (inverse-transform sampling on a 65536-quantile grid; the
 *                 table is built on the Python side with scipy + numpy).
 *   token ids   : out[i] = ((draw >> 32) * vocab) >> 32 (multiply-shift, uniform
 *                 over [0, vocab) up to a 2^-32 bias).
 */
#include <stdint.h>

#define SM_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Start state of the stream for (seed, tensor). */
static inline uint64_t sm_key(uint64_t seed, uint64_t tensor)
{
    return sm_mix(sm_mix(seed + SM_GAMMA) ^ sm_mix(tensor + 0x632be59bd9b4e019ULL));
}

/* The i-th SplitMix64 output of the stream whose state starts at key. */
static inline uint64_t sm_draw(uint64_t key, uint64_t i)
{
    return sm_mix(key + (i + 1) * SM_GAMMA);
}

uint64_t synth_draw(uint64_t seed, uint64_t tensor, uint64_t index)
{
    return sm_draw(sm_key(seed, tensor), index);
}

void synth_table16(uint64_t seed, uint64_t tensor, const uint16_t *table,
                   uint16_t *out, int64_t n, int64_t offset)
{
    const uint64_t key = sm_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = table[sm_draw(key, (uint64_t)(offset + i)) >> 48];
}

void synth_uniform_ids(uint64_t seed, uint64_t tensor, int32_t *out, int64_t n,
                       int64_t offset, uint32_t vocab)
{
    const uint64_t key = sm_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = (int32_t)(((sm_draw(key, (uint64_t)(offset + i)) >> 32) * (uint64_t)vocab) >> 32);
}

/* Fill a constant fp16 pattern (biases = 0, LN gain = 1 in the plain init). */
void synth_fill16(uint16_t *out, int64_t n, uint16_t value)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = value;
}
