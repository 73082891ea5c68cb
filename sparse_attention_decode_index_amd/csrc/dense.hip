// Dense decode over the whole paged cache (gfx950): the dense mode of the
// context-sparsity paper's Fig. 1a, which reads every cached row each step.
//
// Every K/V row of a (b, kv head) serves all G query heads of its group, so
// q K^T is a real [G x 128] x [128 x 16] contraction per page and runs on the
// bf16 MFMA (16x16x32; head rows padded to 16).  The p V product keeps fp32
// weights and runs on the vector ALU: each 16-lane group owns 4 of the page's 16
// rows and 8 of the 128 dims, and reads the weights of its rows from LDS.
// Softmax uses FlashAttention's running (max, sum, accumulator) update (survey
// page, section 5.1).  A workgroup of 4 waves covers 256 pages (4096 tokens), each
// wave 64 pages with the next page's K and V in flight; the 4 wave states are
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

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// grid (splits, num_kv_heads * head_blocks, batch); 256 threads.
// NH = head rows carried per wave (>= heads in this head block, <= 16).
template <int NH>
__global__ __launch_bounds__(kDenseWaves * 64) void dense_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, int num_q_heads, int num_kv_heads,
    int group, int head_blocks, int max_pages, float scale_log2, int splits, float *__restrict__ part_ml,
    float *__restrict__ part_acc)
{
    __shared__ float p_lds[kDenseWaves][kPage][16];           // [token][head]
    __shared__ float a_lds[kDenseWaves][16];                  // rescale factor per head
    __shared__ float w_acc[kDenseWaves][NH][kHeadDim];        // per-wave accumulators for the merge
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

    float mrow[4], lpart[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { mrow[i] = -INFINITY; lpart[i] = 0.f; }
    float acc[NH][8];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[hh][d] = 0.f;

    if (p_begin < p_end) {                                    // wave-uniform; no barriers inside
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
        const int koff = col * kHeadDim + quad * 8;           // MFMA B operand: token col, dims 32 s + 8 quad
        const int voff = quad * kHeadDim + col * 8;           // rows quad + 4 rr, dims 8 col .. +7 (1 KiB rows)

        bf16x8 kb[4];
        u32x4 vw[4];
        {
            const int64_t blk = ((int64_t)__builtin_amdgcn_readlane(pt_lane, 0) * num_kv_heads + g) * (kPage * kHeadDim);
#pragma unroll
            for (int s = 0; s < 4; ++s) kb[s] = *(const bf16x8 *)(kc + blk + koff + 32 * s);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                vw[rr] = __builtin_nontemporal_load((const u32x4 *)(vc + blk + voff + rr * 4 * kHeadDim));
        }

        for (int p = p_begin; p < p_end; ++p) {
            // the next page's K and V are in flight while this one is processed
            bf16x8 kb_n[4];
            u32x4 vw_n[4];
            {
                const int pn = min(p + 1, p_end - 1);
                const int64_t blk =
                    ((int64_t)__builtin_amdgcn_readlane(pt_lane, pn - p_begin) * num_kv_heads + g) * (kPage * kHeadDim);
#pragma unroll
                for (int s = 0; s < 4; ++s) kb_n[s] = *(const bf16x8 *)(kc + blk + koff + 32 * s);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vw_n[rr] = __builtin_nontemporal_load((const u32x4 *)(vc + blk + voff + rr * 4 * kHeadDim));
            }

            f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kb[s], s4, 0, 0, 0);
            const bool tv = p * kPage + col < n;                  // token `col` of this page exists
            float pn_[4], alpha[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = tv ? s4[i] * scale_log2 : -INFINITY;
                const float mx = row16_max(x);                     // finite: the page's first token exists
                const float mn = fmaxf(mrow[i], mx);
                alpha[i] = fast_exp2(mrow[i] - mn);
                pn_[i] = fast_exp2(x - mn);
                mrow[i] = mn;
                lpart[i] = lpart[i] * alpha[i] + pn_[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) p_lds[wave][col][quad * 4 + i] = pn_[i];
            if (col == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) a_lds[wave][quad * 4 + i] = alpha[i];
            }
            wave_sync_lds();
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const float a = a_lds[wave][hh];
#pragma unroll
                for (int d = 0; d < 8; ++d) acc[hh][d] *= a;
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                float vf[8];
                unpack8(vw[rr], vf);
                const float *prow = p_lds[wave][quad + 4 * rr];
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    const float pp = prow[hh];
#pragma unroll
                    for (int d = 0; d < 8; ++d) acc[hh][d] = fmaf(pp, vf[d], acc[hh][d]);
                }
            }
            wave_sync_lds();
#pragma unroll
            for (int s = 0; s < 4; ++s) kb[s] = kb_n[s];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) vw[rr] = vw_n[rr];
        }
    }

    // This wave's state: per head row sums (D layout) and accumulators summed over the
    // 4 lane groups (lanes xor 16 / 32 hold the same dims of different rows).
    float lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] = row16_sum(lpart[i]);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            float a = acc[hh][d];
            a += __shfl_xor(a, 16, 64);
            a += __shfl_xor(a, 32, 64);
            acc[hh][d] = a;
        }
    if (quad == 0) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int d = 0; d < 8; ++d) w_acc[wave][hh][col * 8 + d] = acc[hh][d];
    }
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hm = quad * 4 + i;
            if (hm < NH) { w_ml[wave][hm][0] = mrow[i]; w_ml[wave][hm][1] = lrow[i]; }
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
            A += f * w_acc[w][hh][d];
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
