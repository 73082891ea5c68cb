// Lightweight (reduced-channel) top-k indexer for the decode step (gfx950).
//
// The paper's Fig. 1a routes the sparse decode mode through a lightweight indexer
// that picks the k rows; the German summary (section 3, indexer overhead) costs such
// an indexer with Double Sparsity, and the Sparse Frontier review (section 3.2)
// describes the idea as approximate attention scores from a few key dimensions.
// Here each kv head has a fixed list of kLabelDims = 16 channels (chosen offline by
// calibration); the "label" rows hold those channels of every cached key, 32 B per
// token instead of 256 B, and the indexer ranks tokens by
//     s~_j = sum_{i<16} q[C_g[i]] * K_j[C_g[i]]   (fp32, channel order),
// keeping the exact top-k of s~ (lower index first on equal scores).
//
//  1. label_build_kernel   per (page, kv head): gathers the 16 channels of its 16
//     rows into the label cache [num_pages][Hkv][16][16] bf16 (all pages, or each
//     sequence's current page after an append).
//  2. label_score_kernel   per (b, kv head, 2048 tokens): s~ of the workgroup's
//     tokens for its q heads (16-byte label loads, all in flight; keys stay in the
//     registers of the lane that scored them, their top 15 bits go to LDS), then per
//     head the workgroup's bound (bisection on those codes for the r-th largest of its
//     own scores, r = mu + 6 sqrt(mu) + 8, mu = n_w k / N) and, per 512-token slot,
//     the candidate record (ballot placement in token order) that the exact
//     indexer's select_kernel reads.  Large k: every key to the key rows.
//  3. select_kernel        shared with the exact indexer; its re-scoring fallback
//     recomputes s~ from the label rows.
#include "sdi_device.hpp"
#include "sdi_index.hpp"
#include "sdi_launch.hpp"
#include "sdi_radix.hpp"

namespace sdi {

constexpr int kLabelRowElems = kLabelDims;                    // bf16 per label row
constexpr int kLabelPageElems = kPage * kLabelDims;           // 512 B per (page, kv head)

// grid (ceil(pages / 4), Hkv, B) or (1, Hkv, B) for the current pages only; 256 threads,
// one wave per page: lane (row, part) gathers channels 4 part .. 4 part + 3 of a row.
__global__ __launch_bounds__(256) void label_build_kernel(const uint16_t *__restrict__ kc,
                                                          const int32_t *__restrict__ page_table,
                                                          const int32_t *__restrict__ seq_lens,
                                                          const int32_t *__restrict__ channels, int num_kv_heads,
                                                          int max_pages, int last_only, uint16_t *__restrict__ labels)
{
    const int b = blockIdx.z, g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pages = (seq_lens[b] + kPage - 1) / kPage;
    const int p = last_only ? (wave == 0 ? pages - 1 : -1) : (int)blockIdx.x * 4 + wave;
    if (p < 0 || p >= pages) return;                          // wave-uniform
    const int64_t blk = (int64_t)page_table[(int64_t)b * max_pages + p] * num_kv_heads + g;
    const int row = lane >> 2, part = lane & 3;
    const uint16_t *src = kc + (blk * kPage + row) * kHeadDim;
    const int32_t *ch = channels + g * kLabelDims + 4 * part;
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[ch[i]];
    *(uint2 *)(labels + blk * kLabelPageElems + row * kLabelRowElems + 4 * part) =
        uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
}

// grid (ceil(n_max / (2048 (kTwo ? 2 : 1))), Hkv * head_blocks, B); 256 threads; up to
// kHeads q heads per workgroup.  Wave w owns the workgroup's slot w (tokens 512 w ..
// 512 w + 511), lane l its tokens 512 w + 64 i + l, i = 0..7: it scores them, keeps
// their keys in registers for the records, and shares only their 16-bit codes (for the
// workgroup's bound) in LDS.  A group of at most four heads takes the four-head form:
// half the key registers, which leaves room for a second slot's label rows (kTwo) at
// three workgroups per CU (four without them).
// kTwo: the workgroup also takes the next 2048 tokens, wave w their slot w.  Those
// label rows are put in flight as soon as the first slot is scored, so they arrive
// while the workgroup computes its bound and writes its first records (phases in
// which it would otherwise read nothing); the second slot's tokens are then scored
// and filtered against the same bound directly.
template <bool kAllKeys, int kHeads, bool kTwo>
__global__ __launch_bounds__(kScoreWaves * 64, kHeads <= 4 ? (kTwo ? 3 : 4) : 3)
void label_score_kernel(
    const uint16_t *__restrict__ labels, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, const int32_t *__restrict__ k_per_seq,
    const int32_t *__restrict__ channels, int num_q_heads, int num_kv_heads, int group, int head_blocks,
    int max_pages, int k_max, uint32_t *__restrict__ cand_rec, int slots, uint32_t *__restrict__ keys32,
    int64_t key_stride)
{
    constexpr int kPer = kWaveTokens / 64;                    // 8 tokens per lane
    __shared__ __attribute__((aligned(16))) uint16_t codes[kHeads][kScoreTokensPerBlock];   // 4 KB per head
    __shared__ __attribute__((aligned(16))) float qc_lds[kHeads][kLabelDims];
    __shared__ uint32_t lo_lds[kHeads];
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int n = seq_lens[b];
    const int tok0 = blockIdx.x * kScoreTokensPerBlock * (kTwo ? 2 : 1);
    if (tok0 >= n) return;                                    // whole block exits together
    const int tok1 = tok0 + kScoreTokensPerBlock;             // the second half (kTwo)
    const int kk = min(min(k_per_seq[b], n), k_max);
    const int heads_here = min(kHeads, group - hb * kHeads);
    const int h0 = g * group + hb * kHeads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_wg = min(kScoreTokensPerBlock, n - tok0);     // the workgroup's tokens
    // 1. the lane's 8 label rows in flight (page-table entries, then rows), and the
    //    q values on the head's channels staged in LDS meanwhile (an LDS-only barrier
    //    keeps the rows in flight)
    const bool q_lane = threadIdx.x < heads_here * kLabelDims;   // stages q at one channel of a head
    const int qh = threadIdx.x / kLabelDims, qcn = threadIdx.x - qh * kLabelDims;
    int32_t chan = 0;
    if (q_lane) chan = channels[g * kLabelDims + qcn];
    const int32_t *pt = page_table + (int64_t)b * max_pages;
    int32_t phys[kPer], phys1[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int tl = wave * kWaveTokens + 64 * i + lane;
        phys[i] = pt[(tok0 + min(tl, n_wg - 1)) >> 4];
        if constexpr (kTwo) phys1[i] = pt[min(tok1 + tl, n - 1) >> 4];   // clamped: always a row of it
    }
    uint32_t qbits = 0;
    if (q_lane) qbits = q[((int64_t)b * num_q_heads + h0 + qh) * kHeadDim + chan];
    u32x4 w[kPer][2];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int tl = min(wave * kWaveTokens + 64 * i + lane, n_wg - 1);    // past the row: reload a row of it
        const int64_t row = ((int64_t)phys[i] * num_kv_heads + g) * kPage + (tl & 15);
        const u32x4 *lr = (const u32x4 *)(labels + row * kLabelRowElems);
        w[i][0] = lr[0];
        w[i][1] = lr[1];
    }
    if (q_lane) qc_lds[qh][qcn] = __uint_as_float(qbits << 16);
    lds_barrier();
    uint32_t key[kHeads][kPer];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
        if (h < heads_here) {                                 // uniform
            float qc[kLabelDims];
#pragma unroll
            for (int c = 0; c < kLabelDims; ++c) qc[c] = qc_lds[h][c];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int tl = wave * kWaveTokens + 64 * i + lane;
                key[h][i] = tl < n_wg ? score_key(label_score(qc, w[i][0], w[i][1])) : 0u;
                if constexpr (!kAllKeys) codes[h][tl] = (uint16_t)(key[h][i] >> 17);
            }
        }
    }
    // the second slot's label rows, in flight from here on (every lane loads: a row
    // past the sequence is replaced by its last row and not scored)
    u32x4 w1[kPer][2];
    if constexpr (kTwo) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = min(tok1 + wave * kWaveTokens + 64 * i + lane, n - 1);
            const int64_t row = ((int64_t)phys1[i] * num_kv_heads + g) * kPage + (t & 15);
            const u32x4 *lr = (const u32x4 *)(labels + row * kLabelRowElems);
            w1[i][0] = lr[0];
            w1[i][1] = lr[1];
        }
    }
    if constexpr (kAllKeys) {                                 // every key to the head's key row
#pragma unroll
        for (int h = 0; h < kHeads; ++h) {
            if (h < heads_here) {
                uint32_t *krow = keys32 + ((int64_t)b * num_q_heads + h0 + h) * key_stride + tok0;
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int tl = wave * kWaveTokens + 64 * i + lane;
                    if (tl < n_wg) krow[tl] = key[h][i];
                }
                if constexpr (kTwo) {
                    float qc[kLabelDims];
#pragma unroll
                    for (int c = 0; c < kLabelDims; ++c) qc[c] = qc_lds[h][c];
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const int tl = kScoreTokensPerBlock + wave * kWaveTokens + 64 * i + lane;
                        if (tok0 + tl < n) krow[tl] = score_key(label_score(qc, w1[i][0], w1[i][1]));
                    }
                }
            }
        }
        return;
    } else {
        lds_barrier();                                        // codes complete (loads stay in flight)
        // 2. per head (one wave each): the r-th largest code of the workgroup's own keys
        for (int hh = wave; hh < heads_here; hh += kScoreWaves) {
            uint32_t b_lo = 0xFFFFFFFFu;                      // k' = 0 or N: no candidates needed
            if (kk > 0 && kk < n) {
                const float mu = (float)n_wg * (float)kk / (float)n;
                const uint32_t r = (uint32_t)ceilf(mu + 6.f * sqrtf(mu) + 8.f);
                b_lo = 0u;                                    // a small workgroup keeps everything
                if (r < (uint32_t)n_wg) {
                    // the lane's 32 codes, two per word (16-byte reads).  A code is the
                    // top 15 bits of a key, so code >= mid is bit 15 of (code | 0x8000) - mid:
                    // two compares per subtract, counted by bit count
                    constexpr int words = kScoreTokensPerBlock / 64 / 2;
                    uint32_t cw[words];
#pragma unroll
                    for (int v = 0; v < words / 4; ++v) {
                        const u32x4 w4 = *(const u32x4 *)&codes[hh][lane * 2 * words + 8 * v];
                        cw[4 * v + 0] = w4.x | 0x80008000u; cw[4 * v + 1] = w4.y | 0x80008000u;
                        cw[4 * v + 2] = w4.z | 0x80008000u; cw[4 * v + 3] = w4.w | 0x80008000u;
                    }
                    uint32_t lo_c = 0, hi_c = 0x8000;         // count(code >= lo_c) >= r > count(code >= hi_c)
                    while (hi_c - lo_c > 1) {
                        const uint32_t mid = (lo_c + hi_c) >> 1, mid2 = mid | (mid << 16);
                        uint32_t m0 = 0, m1 = 0;
#pragma unroll
                        for (int e = 0; e < words; e += 2) {
                            m0 += __popc((cw[e] - mid2) & 0x80008000u);
                            m1 += __popc((cw[e + 1] - mid2) & 0x80008000u);
                        }
                        if (wave_total(m0 + m1) >= r) lo_c = mid; else hi_c = mid;
                    }
                    b_lo = lo_c << 17;
                }
            }
            if (lane == 0) lo_lds[hh] = b_lo;
        }
        lds_barrier();
        // 3. the records: wave w writes slot w of each head straight from its registers;
        //    candidates (keys >= the bound) are placed in token order by ballot; a store
        //    past the record's 192 entries (an overflowed slot) aims past the row and is
        //    dropped by the buffer range check, and the header marks the overflow
        const int s_tok0 = tok0 + wave * kWaveTokens;
        if (s_tok0 >= n) return;                              // wave-uniform
        const int slot = s_tok0 / kWaveTokens;
        const uint32_t row_bytes = (uint32_t)slots * kRecWords * 4u;
        const uint32_t rec0 = (uint32_t)slot * kRecWords * 4u;
#pragma unroll
        for (int h = 0; h < kHeads; ++h) {
            if (h < heads_here) {
                const uint32_t lo = lo_lds[h];
                const int64_t row_h = (int64_t)b * num_q_heads + h0 + h;
                const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                    cand_rec + row_h * slots * kRecWords, 0, (int)row_bytes, kBufferDword3);
                uint32_t cnt = 0, kmax = 0;
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int tl = wave * kWaveTokens + 64 * i + lane;
                    const bool take = tl < n_wg && key[h][i] >= lo;
                    const uint64_t m = __ballot(take);
                    const uint32_t pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    const bool put = take && pos < (uint32_t)kCandCap;
                    __builtin_amdgcn_raw_buffer_store_b32(key[h][i], rsrc, put ? rec0 + 4u * pos : kDropOffset, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(64 * i + lane), rsrc,
                                                          put ? rec0 + (kCandCap + 4) * 4u + 2u * pos : kDropOffset,
                                                          0, 0);
                    kmax = max(kmax, take ? key[h][i] : 0u);
                    cnt += (uint32_t)__popcll(m);
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
                const u32x4 hdr = u32x4{cnt > (uint32_t)kCandCap ? kCandOverflow : cnt, lo, kmax, 0u};
                __builtin_amdgcn_raw_buffer_store_b128(hdr, rsrc, lane == 0 ? rec0 + kCandCap * 4u : kDropOffset, 0, 0);
            }
        }
        // 4. the second slot (kTwo): scored from the rows in flight and filtered
        //    against the same bounds, its record written the same way
        if constexpr (kTwo) {
            const int s1_tok0 = tok1 + wave * kWaveTokens;
            if (s1_tok0 >= n) return;                         // wave-uniform
            const uint32_t rec1 = (uint32_t)(s1_tok0 / kWaveTokens) * kRecWords * 4u;
#pragma unroll
            for (int h = 0; h < kHeads; ++h) {
                if (h < heads_here) {
                    float qc[kLabelDims];
#pragma unroll
                    for (int c = 0; c < kLabelDims; ++c) qc[c] = qc_lds[h][c];
                    const uint32_t lo = lo_lds[h];
                    const int64_t row_h = (int64_t)b * num_q_heads + h0 + h;
                    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                        cand_rec + row_h * slots * kRecWords, 0, (int)row_bytes, kBufferDword3);
                    uint32_t cnt = 0, kmax = 0;
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const bool valid = s1_tok0 + 64 * i + lane < n;
                        const uint32_t k1 = valid ? score_key(label_score(qc, w1[i][0], w1[i][1])) : 0u;
                        const bool take = valid && k1 >= lo;
                        const uint64_t m = __ballot(take);
                        const uint32_t pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        const bool put = take && pos < (uint32_t)kCandCap;
                        __builtin_amdgcn_raw_buffer_store_b32(k1, rsrc, put ? rec1 + 4u * pos : kDropOffset, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(64 * i + lane), rsrc,
                                                              put ? rec1 + (kCandCap + 4) * 4u + 2u * pos : kDropOffset,
                                                              0, 0);
                        kmax = max(kmax, take ? k1 : 0u);
                        cnt += (uint32_t)__popcll(m);
                    }
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
                    const u32x4 hdr = u32x4{cnt > (uint32_t)kCandCap ? kCandOverflow : cnt, lo, kmax, 0u};
                    __builtin_amdgcn_raw_buffer_store_b128(hdr, rsrc, lane == 0 ? rec1 + kCandCap * 4u : kDropOffset,
                                                           0, 0);
                }
            }
        }
    }
}

// ---- host side ---------------------------------------------------------------------------

size_t label_bytes(int num_pages, int num_kv_heads)
{
    return (size_t)num_pages * num_kv_heads * kLabelPageElems * sizeof(uint16_t);
}

hipError_t launch_label_build(const LabelArgs &a, int last_only, hipStream_t stream)
{
    const int bx = last_only ? 1 : (a.max_pages + 3) / 4;
    hipLaunchKernelGGL(label_build_kernel, dim3(bx, a.num_kv_heads, a.batch), dim3(256), 0, stream,
                       (const uint16_t *)a.k_cache, a.page_table, a.seq_lens, a.channels, a.num_kv_heads,
                       a.max_pages, last_only, (uint16_t *)a.labels);
    return hipGetLastError();
}

hipError_t launch_label_index_topk(const LabelArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int heads = group <= 4 ? 4 : kHeadBlock;             // q heads per workgroup
    const int head_blocks = (group + heads - 1) / heads;
    const int64_t stride = (int64_t)index_topk_key_stride(a.n_max);
    const int slots = index_topk_slots(a.n_max);
    uint32_t *keys32 = (uint32_t *)a.ws;
    uint32_t *cand_rec = keys32 + (size_t)a.batch * a.num_q_heads * stride;
    const SelectPlan plan = plan_select(a.k_max, a.n_max, slots);
    // The four-head form also takes a second slot per wave (measured faster there:
    // 39.0 -> 37.5 us on the 8 x 32 x 32768 layer); the eight-head form would drop
    // to two workgroups per CU with it and measured slower.
    const bool two = heads == 4;
    const int per_block = (two ? 2 : 1) * kScoreTokensPerBlock;
    const dim3 grid((a.n_max + per_block - 1) / per_block, a.num_kv_heads * head_blocks, a.batch);
    auto launch_score = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kScoreWaves * 64), 0, stream, (const uint16_t *)a.labels,
                           a.page_table, a.seq_lens, (const uint16_t *)a.q, a.k_per_seq, a.channels, a.num_q_heads,
                           a.num_kv_heads, group, head_blocks, a.max_pages, a.k_max, cand_rec, slots, keys32, stride);
    };
    if (two) {
        if (plan.all_keys) launch_score(label_score_kernel<true, 4, true>);
        else launch_score(label_score_kernel<false, 4, true>);
    } else {
        if (plan.all_keys) launch_score(label_score_kernel<true, kHeadBlock, false>);
        else launch_score(label_score_kernel<false, kHeadBlock, false>);
    }
    SelectArgs s{(const uint16_t *)a.k_cache, a.page_table, a.seq_lens, a.k_per_seq, (const uint16_t *)a.q,
                 cand_rec, slots, plan.cap, plan.all_keys ? 1 : 0, keys32, stride, a.num_q_heads, a.num_kv_heads,
                 group, a.max_pages, a.k_max, a.idx_out, (const uint16_t *)a.labels, a.channels};
    return launch_select(s, plan, a.batch, stream);
}

}  // namespace sdi
