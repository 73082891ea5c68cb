// Dense decode over the whole paged cache (gfx950): the dense mode of the
// context-sparsity paper's Fig. 1a, which reads every cached row each step.
//
// Every K/V row of a (b, kv head) serves all G query heads of its group, so both
// products are real contractions over the group and run on the bf16 MFMA
// (16x16x32, head rows padded to 16): q K^T ([G x 128] x [128 x 32 tokens]) and
// P V ([G x 32 tokens] x [32 x 128]), the weights P rounded to bf16.  V's rows are
// transposed into the MFMA operand through LDS.  Softmax uses FlashAttention's
// running (max, sum, accumulator) update (survey page, section 5.1).  A workgroup of
// 4 waves covers 256 pages (4096 tokens), each wave 64 pages, two at a time with the
// next two pages' K and V in flight; the 4 wave states are
// merged in LDS into one partial per workgroup, and the partials of a sequence are
// combined by the same log-sum-exp merge as the sparse path.
#include "sdi_device.hpp"
#include "sdi_launch.hpp"

namespace sdi {

constexpr int kDenseWaves = 4;
// 64 pages per wave (one page-table entry per lane), 4096 tokens per partial.  Against
// 16 pages (1024 tokens) this writes a quarter of the partials and merges a quarter:
// 172 / 348 / 1282 / 1871 us instead of 184 / 382 / 1374 / 1933 us on the Llama-3-8B
// layer, the long-retrieval batch, the sweep and the agentic batch.
constexpr int kDensePagesPerWave = 64;
constexpr int kDenseTokensPerSplit = kDenseWaves * kDensePagesPerWave * kPage;   // 4096 tokens per partial
static_assert(kDensePagesPerWave <= 64, "one page-table entry per lane");
constexpr float kDenseLog2e = 1.4426950408889634f;


// LDS tiles of a wave: the V rows of two pages (32 tokens x 128 dims, bf16, rows of
// 132 values: 264 B, 8-byte aligned) and the bf16 weights P[head][token] of those 32
// tokens (rows of 40 values).  The row strides put the transposed operand reads in
// different banks: V row r + 8 starts 16 banks after row r, so the four 16-lane groups
// of a read (tokens 8 quad + e) cover disjoint banks; P rows of the 16 heads start 20
// banks apart.
constexpr int kVStride = kHeadDim + 4;
constexpr int kPStride = 2 * kPage + 8;
constexpr int kVTile = 2 * kPage * kVStride;                  // bf16 values per wave
constexpr int kPTile = 16 * kPStride;

// bf16 bits of a finite fp32 value, round to nearest even
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// grid (splits, num_kv_heads * head_blocks, batch); 256 threads.
// NH = head rows kept for the merge (>= heads in this head block, <= 16).
//
// Per wave and per pair of pages (32 tokens): S = q K^T on 8 MFMAs (A = q, 16 head
// rows; B = K, one token per column) gives lane (col, quad) the scores of token col
// for heads 4 quad + i.  The running max, the rescale factor and the weights follow
// the online softmax per head; the weights are rounded to bf16, and the row sums
// accumulate those rounded weights, so numerator and denominator use the same values.
// The weights go to LDS as P[head][token] and the V rows as [token][dim]; then
// O += P V runs on 8 more MFMAs (A = P: head col, tokens 8 quad .. +7; B = V: tokens
// 8 quad .. +7, dim col + 16 j), and lane (col, quad) ends with O[heads 4 quad + i]
// [dims col + 16 j].  The next pair's K and V are in flight meanwhile.
template <int NH>
__global__ __launch_bounds__(kDenseWaves * 64) void dense_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, int num_q_heads, int num_kv_heads,
    int group, int head_blocks, int max_pages, float scale_log2, int splits, float *__restrict__ part_ml,
    float *__restrict__ part_acc)
{
    static_assert(NH * kHeadDim * 4 <= kVTile * 2, "the merge rows fit a wave's V tile");
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[kDenseWaves][kVTile];
    __shared__ __attribute__((aligned(16))) uint16_t p_lds[kDenseWaves][kPTile];
    __shared__ float w_ml[kDenseWaves][NH][2];
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    const int n = seq_lens[b];
    const int pages_seq = (n + kPage - 1) / kPage;
    const int split = blockIdx.x;
    if (split * kDenseWaves * kDensePagesPerWave >= pages_seq) return;   // whole block exits together
    const int p_begin = (split * kDenseWaves + wave) * kDensePagesPerWave;
    const int p_end = min(p_begin + kDensePagesPerWave, pages_seq);
    const int heads_here = min(16, group - hb * 16);
    const int h0 = g * group + hb * 16;
    uint16_t *vt = v_lds[wave];
    uint16_t *pt_w = p_lds[wave];

    float mrow[4], lpart[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { mrow[i] = -INFINITY; lpart[i] = 0.f; }
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (p_begin < p_end) {                                    // wave-uniform; no workgroup barriers inside
        bf16x8 qa[4];
        {
            const bool live = col < heads_here;
            const bf16x8 *qrow =
                (const bf16x8 *)(q + ((int64_t)b * num_q_heads + h0 + (live ? col : 0)) * kHeadDim);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qa[s] = live ? qrow[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
        const int32_t *pt = page_table + (int64_t)b * max_pages;
        const int pt_lane = (p_begin + lane < p_end) ? pt[p_begin + lane] : 0;   // the wave's entries, one per lane
        const int koff = col * kHeadDim + quad * 8;           // K operand: token col, dims 32 s + 8 quad
        const int voff = quad * kHeadDim + col * 8;           // V rows quad + 4 rr, dims 8 col .. +7

        // K and V of pages p, p + 1 (a page past the wave's range re-reads its last page;
        // its tokens are masked below)
        auto load_pair = [&](int p, bf16x8 (&kb)[2][4], u32x4 (&vw)[2][4]) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int pg = min(p + pp, p_end - 1);
                const int64_t blk =
                    ((int64_t)__builtin_amdgcn_readlane(pt_lane, pg - p_begin) * num_kv_heads + g) * (kPage * kHeadDim);
#pragma unroll
                for (int s = 0; s < 4; ++s) kb[pp][s] = *(const bf16x8 *)(kc + blk + koff + 32 * s);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vw[pp][rr] = __builtin_nontemporal_load((const u32x4 *)(vc + blk + voff + rr * 4 * kHeadDim));
            }
        };
        bf16x8 kb[2][4];
        u32x4 vw[2][4];
        load_pair(p_begin, kb, vw);

        for (int p = p_begin; p < p_end; p += 2) {
            bf16x8 kb_n[2][4];
            u32x4 vw_n[2][4];
            load_pair(min(p + 2, p_end - 1), kb_n, vw_n);     // the next pair, in flight

            f32x4 s4[2];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                s4[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) s4[pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kb[pp][s], s4[pp], 0, 0, 0);
            }
            float alpha[4], w[2][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x[2];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const bool tv = (p + pp < p_end) && (p + pp) * kPage + col < n;   // token col of page p + pp
                    x[pp] = tv ? s4[pp][i] * scale_log2 : -INFINITY;
                }
                const float mx = fmaxf(row16_max(x[0]), row16_max(x[1]));   // finite: page p's first token exists
                const float mn = fmaxf(mrow[i], mx);
                alpha[i] = fast_exp2(mrow[i] - mn);
                float ls = 0.f;
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const uint32_t wb = bf16_bits_rne(fast_exp2(x[pp] - mn));
                    w[pp][i] = __uint_as_float(wb << 16);
                    ls += w[pp][i];
                    pt_w[(4 * quad + i) * kPStride + kPage * pp + col] = (uint16_t)wb;
                }
                mrow[i] = mn;
                lpart[i] = lpart[i] * alpha[i] + ls;
            }
            // V rows of the pair to LDS: row 16 pp + quad + 4 rr, dims 8 col .. +7 (two 8-byte writes)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    uint2 *dst = (uint2 *)(vt + (kPage * pp + quad + 4 * rr) * kVStride + 8 * col);
                    dst[0] = uint2{vw[pp][rr].x, vw[pp][rr].y};
                    dst[1] = uint2{vw[pp][rr].z, vw[pp][rr].w};
                }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
            wave_lds_sync();
            const bf16x8 pa = *(const bf16x8 *)(pt_w + col * kPStride + 8 * quad);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint16_t *src = vt + 8 * quad * kVStride + col + 16 * j;
                u32x4 vb;
                vb.x = (uint32_t)src[0 * kVStride] | ((uint32_t)src[1 * kVStride] << 16);
                vb.y = (uint32_t)src[2 * kVStride] | ((uint32_t)src[3 * kVStride] << 16);
                vb.z = (uint32_t)src[4 * kVStride] | ((uint32_t)src[5 * kVStride] << 16);
                vb.w = (uint32_t)src[6 * kVStride] | ((uint32_t)src[7 * kVStride] << 16);
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[j], 0, 0, 0);
            }
            wave_lds_sync();                                  // tiles free for the next pair
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
                for (int s = 0; s < 4; ++s) kb[pp][s] = kb_n[pp][s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) vw[pp][rr] = vw_n[pp][rr];
            }
        }
    }

    // This wave's state: per head row sums, and O straight from the MFMA layout into the
    // wave's own V tile, reused as its [head][dim] merge rows.
    float *w_acc = (float *)vt;
    float lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] = row16_sum(lpart[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hm = quad * 4 + i;
        if (hm < NH) {
#pragma unroll
            for (int j = 0; j < 8; ++j) w_acc[hm * kHeadDim + col + 16 * j] = o[j][i];
            if (col == 0) { w_ml[wave][hm][0] = mrow[i]; w_ml[wave][hm][1] = lrow[i]; }
        }
    }
    __syncthreads();

    // Merge the 4 waves: one partial (m, l, acc[128]) per head for this split.
    const int64_t bh0 = (int64_t)b * num_q_heads + h0;
    for (int t = threadIdx.x; t < heads_here * kHeadDim; t += kDenseWaves * 64) {
        const int hh = t / kHeadDim, d = t - hh * kHeadDim;
        float M = w_ml[0][hh][0];
#pragma unroll
        for (int w = 1; w < kDenseWaves; ++w) M = fmaxf(M, w_ml[w][hh][0]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < kDenseWaves; ++w) {
            const float f = (M == -INFINITY) ? 0.f : fast_exp2(w_ml[w][hh][0] - M);
            L += f * w_ml[w][hh][1];
            A += f * ((const float *)v_lds[w])[hh * kHeadDim + d];
        }
        const int64_t ps = (bh0 + hh) * splits + split;
        part_acc[ps * kHeadDim + d] = A;
        if (d == 0) { part_ml[ps * 2] = M; part_ml[ps * 2 + 1] = L; }
    }
}

int dense_splits(int n_max) { return (n_max + kDenseTokensPerSplit - 1) / kDenseTokensPerSplit; }

size_t dense_workspace_bytes(int batch, int num_q_heads, int n_max)
{
    return (size_t)batch * num_q_heads * dense_splits(n_max) * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_dense(const AttendArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int head_blocks = (group + 15) / 16;
    const int heads_max = std::min(16, group);
    const int splits = dense_splits(a.n_max);
    const size_t bhs = (size_t)a.batch * a.num_q_heads * splits;
    float *part_acc = (float *)a.ws;
    float *part_ml = part_acc + bhs * kHeadDim;
    dim3 grid(splits, a.num_kv_heads * head_blocks, a.batch);
    const float sl2 = a.scale * kDenseLog2e;
#define SDI_DENSE_LAUNCH(NH)                                                                                     \
    hipLaunchKernelGGL(dense_kernel<NH>, grid, dim3(kDenseWaves * 64), 0, stream, (const uint16_t *)a.k_cache,  \
                       (const uint16_t *)a.v_cache, a.page_table, a.seq_lens, (const uint16_t *)a.q,           \
                       a.num_q_heads, a.num_kv_heads, group, head_blocks, a.max_pages, sl2, splits, part_ml,   \
                       part_acc)
    if (heads_max <= 4)
        SDI_DENSE_LAUNCH(4);
    else if (heads_max <= 8)
        SDI_DENSE_LAUNCH(8);
    else
        SDI_DENSE_LAUNCH(16);
#undef SDI_DENSE_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(part_ml, part_acc, splits, kDenseTokensPerSplit, a.seq_lens, a.n_max, a.batch,
                        a.num_q_heads, a.out, stream);
}

}  // namespace sdi
