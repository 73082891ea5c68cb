/*
 * Seeded, counter-based synthetic inputs for the context-sparse decode
 * workloads (bf16 queries and a paged bf16 KV cache).
 *
 * This file holds random-number generation and data placement only; it
 * computes nothing of the attention method itself.  Both the CPU oracle and
 * the GPU library consume what it writes, so it shares code with neither.
 *
 * Every value is a pure function of (seed, tag, counter), so a tensor can be
 * generated in any order, in pieces, or under any physical page layout and
 * still hold the same logical contents.
 *
 * Generator: the splitmix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
 * in Vigna's public splitmix64) applied to base + (counter + 1) * golden-gamma.
 * Normals: Box-Muller (cosine branch only, one normal per counter).
 * Student-t with 3 degrees of freedom: z0 / sqrt((z1^2 + z2^2 + z3^2) / 3).
 * fp32 -> bf16 conversion rounds to nearest even (no NaN is ever produced).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Per-stream base: the seed and a 64-bit tag that names the tensor slice. */
static inline uint64_t stream_base(uint64_t seed, uint64_t tag)
{
    return mix64(mix64(seed + SYNTH_GOLDEN) ^ (tag * 0xD1B54A32D192ED03ULL + 0x8CB92BA72F3D8DD7ULL));
}

static inline uint64_t draw(uint64_t base, uint64_t ctr)
{
    return mix64(base + (ctr + 1ULL) * SYNTH_GOLDEN);
}

/* 53-bit uniforms: (0, 1] and [0, 1). */
static inline double unit_open0(uint64_t x) { return (double)((x >> 11) + 1ULL) * 0x1.0p-53; }
static inline double unit_closed0(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t base, uint64_t ctr)
{
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = unit_open0(draw(base, 2ULL * ctr));
    double u2 = unit_closed0(draw(base, 2ULL * ctr + 1ULL));
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline double student_t3_at(uint64_t base, uint64_t ctr)
{
    double z0 = normal_at(base, 4ULL * ctr + 0ULL);
    double z1 = normal_at(base, 4ULL * ctr + 1ULL);
    double z2 = normal_at(base, 4ULL * ctr + 2ULL);
    double z3 = normal_at(base, 4ULL * ctr + 3ULL);
    double chi = (z1 * z1 + z2 * z2 + z3 * z3) / 3.0;
    return z0 / sqrt(chi);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Tag layout: tensor (8 bits) | step (16) | batch row (20) | head (20). */
uint64_t synth_tag(uint32_t tensor, uint32_t step, uint32_t b, uint32_t head)
{
    return ((uint64_t)(tensor & 0xFFu) << 56) | ((uint64_t)(step & 0xFFFFu) << 40) |
           ((uint64_t)(b & 0xFFFFFu) << 20) | (uint64_t)(head & 0xFFFFFu);
}

/* Raw 64-bit draws (used for seeded permutations and positions). */
void synth_u64(uint64_t seed, uint64_t tag, uint64_t ctr0, int64_t n, uint64_t *out)
{
    uint64_t base = stream_base(seed, tag);
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw(base, ctr0 + (uint64_t)i);
}

/* n values of scale * N(0,1), rounded to bf16, at counters ctr0 .. ctr0+n-1. */
void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t ctr0, int64_t n, float scale,
                       uint16_t *out)
{
    uint64_t base = stream_base(seed, tag);
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne((float)(scale * normal_at(base, ctr0 + (uint64_t)i)));
}

/* Same, as fp64 (for building planted keys before rounding). */
void synth_normal_f64(uint64_t seed, uint64_t tag, uint64_t ctr0, int64_t n, double *out)
{
    uint64_t base = stream_base(seed, tag);
    for (int64_t i = 0; i < n; ++i)
        out[i] = normal_at(base, ctr0 + (uint64_t)i);
}

/* Round fp64 values to bf16 (through fp32). */
void synth_round_bf16(const double *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne((float)in[i]);
}

/* Logical value of one K or V element: token n, channel d of (b, kv head g).
 * Channels flagged in the outlier mask draw outlier_scale * t3 from a stream
 * of their own; the rest draw N(0,1). */
static inline uint16_t kv_value(uint64_t base_n, uint64_t base_t, int outlier, float outlier_scale,
                                uint64_t ctr)
{
    double v = outlier ? (double)outlier_scale * student_t3_at(base_t, ctr) : normal_at(base_n, ctr);
    return f32_to_bf16_rne((float)v);
}

/*
 * Fill tokens [lo[b], hi[b]) of every (b, kv head) into a paged cache laid out
 * [num_pages][num_kv_heads][page_size][head_dim], using page_table
 * [batch][max_pages].  Slots outside the filled ranges are left untouched.
 * outlier_mask is [batch][num_kv_heads][head_dim] bytes (nonzero = outlier
 * channel) or NULL.  Parallel over (b, kv head, page).
 */
void synth_fill_kv_paged(uint64_t seed, uint32_t tensor, int32_t batch, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_size, int32_t max_pages,
                         const int32_t *page_table, const int32_t *lo, const int32_t *hi,
                         const uint8_t *outlier_mask, float outlier_scale, uint16_t *cache)
{
    int64_t total = (int64_t)batch * num_kv_heads * max_pages;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; ++w) {
        int32_t lp = (int32_t)(w % max_pages);
        int32_t g = (int32_t)((w / max_pages) % num_kv_heads);
        int32_t b = (int32_t)(w / ((int64_t)max_pages * num_kv_heads));
        int32_t t0 = lp * page_size, t1 = t0 + page_size;
        if (t0 < lo[b]) t0 = lo[b];
        if (t1 > hi[b]) t1 = hi[b];
        if (t0 >= t1) continue;
        int64_t phys = page_table[(int64_t)b * max_pages + lp];
        uint64_t base_n = stream_base(seed, synth_tag(tensor, 0, (uint32_t)b, (uint32_t)g));
        uint64_t base_t = stream_base(seed, synth_tag(tensor | 0x80u, 0, (uint32_t)b, (uint32_t)g));
        const uint8_t *mask = outlier_mask ? outlier_mask + ((int64_t)b * num_kv_heads + g) * head_dim : 0;
        for (int32_t n = t0; n < t1; ++n) {
            uint16_t *row = cache + ((phys * num_kv_heads + g) * page_size + (n % page_size)) * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) {
                uint64_t ctr = (uint64_t)n * (uint64_t)head_dim + (uint64_t)d;
                row[d] = kv_value(base_n, base_t, mask ? mask[d] != 0 : 0, outlier_scale, ctr);
            }
        }
    }
}

/* The rows of token tok[b] for every (b, kv head), same values as the paged
 * fill would place there: out is [batch][num_kv_heads][head_dim]. */
void synth_kv_rows(uint64_t seed, uint32_t tensor, int32_t batch, int32_t num_kv_heads,
                   int32_t head_dim, const int32_t *tok, const uint8_t *outlier_mask,
                   float outlier_scale, uint16_t *out)
{
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t g = 0; g < num_kv_heads; ++g) {
            uint64_t base_n = stream_base(seed, synth_tag(tensor, 0, (uint32_t)b, (uint32_t)g));
            uint64_t base_t = stream_base(seed, synth_tag(tensor | 0x80u, 0, (uint32_t)b, (uint32_t)g));
            const uint8_t *mask = outlier_mask ? outlier_mask + ((int64_t)b * num_kv_heads + g) * head_dim : 0;
            uint16_t *row = out + ((int64_t)b * num_kv_heads + g) * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) {
                uint64_t ctr = (uint64_t)tok[b] * (uint64_t)head_dim + (uint64_t)d;
                row[d] = kv_value(base_n, base_t, mask ? mask[d] != 0 : 0, outlier_scale, ctr);
            }
        }
}

/* Queries of one decode step: out is [batch][num_q_heads][head_dim]. */
void synth_queries(uint64_t seed, uint32_t step, int32_t batch, int32_t num_q_heads,
                   int32_t head_dim, uint16_t *out)
{
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t h = 0; h < num_q_heads; ++h)
            synth_normal_bf16(seed, synth_tag(1u, step, (uint32_t)b, (uint32_t)h), 0, head_dim, 1.0f,
                              out + ((int64_t)b * num_q_heads + h) * head_dim);
}
