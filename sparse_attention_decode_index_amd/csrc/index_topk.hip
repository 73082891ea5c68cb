// Exact top-k indexer for the context-sparse decode step (gfx950).
//
// The selection is the exact "oracle top-k" of the context-sparsity paper
// (German technical summary, section 2, sparsity mechanisms): for each
// (sequence, query head) keep the k tokens with the largest raw score q . K_j,
// lower index first on equal scores, per query head (paper section 1).
//
// Scores are fp32 sums of bf16 products from one MFMA instruction sequence; a
// score's order-preserving uint32 key is its rank key.  Two launches:
//
//  1. score_kernel   streams every K page once per (b, kv head) with contiguous
//                    non-temporal 1 KiB loads, transposes each page through LDS
//                    into the MFMA operand layout and scores 16 tokens x up to 8
//                    heads of the GQA group per 4 MFMAs (16x16x32 bf16).  Each
//                    workgroup (4 waves, 2048 tokens, two per CU) first scores 16
//                    pages per wave (1024 tokens per head),
//                    keeps those keys in registers and takes, per head, a sample
//                    order statistic a safe margin above its share of the k-th key:
//                    a lower bound `lo` that about 1.5..2.5 k tokens of the row
//                    reach.  Only the tokens whose key reaches `lo` leave the chip:
//                    (key, position) pairs, appended in token order to a per-wave
//                    LDS list and written once per 512-token slot with the slot's
//                    bound.  HBM writes interleaved with the K stream cost several
//                    times their size in read bandwidth, so writing a few percent of
//                    the tokens instead of a code per token keeps the pass at
//                    streaming speed.
//  2. select_kernel  per (b, h): the slot counts give each candidate's place, the
//                    candidates are gathered into LDS in token order, radix passes
//                    over key - min(lo) (kHistBits at a time, usually two) find the
//                    exact k-th key T and an ordered compaction writes the row.
//
// Exactness does not depend on the sample: if T, the k'-th largest candidate key,
// is at least every workgroup's bound, then every token left out (its key is below
// its workgroup's bound) is below T, so the candidates hold every token that can be
// selected, ties included.  When that check fails, or a slot's list overflows, or
// the row has more candidates than LDS holds, the select re-scores the whole row to
// 32-bit keys in the workspace (same MFMA sequence, bit-identical keys) and
// radix-selects over them.
#include "sdi_device.hpp"
#include "sdi_launch.hpp"
#include "sdi_radix.hpp"
#include "sdi_index.hpp"

#include <cmath>
#include <type_traits>

namespace sdi {

// ---- score pass --------------------------------------------------------------------------
constexpr int kScoreUnroll = 2;                               // pages per register buffer (a group)
constexpr int kScoreBufs = 2;                                 // groups in flight per wave (3 measured no faster)
constexpr int kSlotGroups = kScorePagesPerWave / kScoreUnroll;
constexpr int kGatherUnroll = 4;                              // candidates in flight per select thread
constexpr int kStageRow = kRowBytes + 16;                     // padded LDS row: conflict-free both ways
constexpr int kStagePage = kPage * kStageRow;                 // 4352 B
constexpr int kSubCap = kCandCap / 4;                         // ... as 4 lane lists (one per quad) of 48
constexpr int kSubStride = kSubCap + 1;                       // entries of a list, with its pad slot
constexpr int kLists = kHeadBlock * 4;                        // lane lists of a wave (head, quad)
constexpr int kSamplePagesPerWave = 16;                       // the first pages of each wave ...
constexpr int kBlockSample = kScoreWaves * kSamplePagesPerWave * kPage;   // ... 1024 tokens per head
constexpr int kSampStride = kBlockSample + 16;
// Sample codes of head h start at h * kSampStride: the pad (16 codes, 8 banks) puts the
// head rows of one write 8 banks apart, so the 32 head lanes of a page write (8 heads x 4
// quads, 2 banks apart within a head) all land in different banks.
constexpr int kSampleGroups = kSamplePagesPerWave / kScoreUnroll;
static_assert(kSampleGroups % 2 == 0 && kSamplePagesPerWave <= kScorePagesPerWave, "sample = pairs of groups");


// ---- select ------------------------------------------------------------------------------
// MFMA B operand for the q rows of a head block: lane (col, quad) holds head col's
// dims 32 s + 8 quad .. +7 (zeros for heads past the block).
__device__ __forceinline__ void load_q_operand(bf16x8 (&qb)[4], const uint16_t *__restrict__ q, int64_t row0,
                                               int heads_here, int col, int quad)
{
    const bool live = col < heads_here;
    const bf16x8 *qrow = (const bf16x8 *)(q + (row0 + (live ? col : 0)) * kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        qb[s] = live ? qrow[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// The score MFMA sequence: D[token 4 quad + i][head col] for 16 tokens (A: row col,
// dims 32 s + 8 quad) and up to 16 heads (B).  Every score in this file comes from
// this function, so that keys agree bit for bit wherever they are computed.
__device__ __forceinline__ f32x4 score_mfma(const bf16x8 (&ka)[4], const bf16x8 (&qb)[4])
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[s], acc, 0, 0, 0);
    return acc;
}

// Scores of up to 16 tokens of one head block: the 16 K rows (cache row number per
// lane `col`, or -1) loaded straight into the A layout, the block's q as B.  Lanes
// with col == head-in-block get the scores of tokens 4 quad .. +3.
__device__ __forceinline__ f32x4 rescore16(const uint16_t *__restrict__ kc, int row, const bf16x8 (&qb)[4],
                                          int quad)
{
    bf16x8 ka[4];
    const bf16x8 *src = (const bf16x8 *)(kc + (int64_t)(row < 0 ? 0 : row) * kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        ka[s] = row >= 0 ? src[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    return score_mfma(ka, qb);
}

// Keeps the instruction scheduler from moving anything across this point: the
// score pass relies on program order (stage a group, put the next group in flight,
// then score) so that each wait covers only the group being staged.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// f(integral_constant<int, i>) for i = B .. E - 1, in order, at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}



// ---- 1. score pass -----------------------------------------------------------------------

// grid (ceil(n_max / 2048), kv_heads * head_blocks, batch); 256 threads.
template <int kSlots, bool kAllKeys>
__global__ __launch_bounds__(kScoreWaves * 64, 2) void score_kernel(
    const uint16_t *__restrict__ kc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, const int32_t *__restrict__ k_per_seq,
    int num_q_heads, int num_kv_heads, int group, int head_blocks, int max_pages, int k_max,
    uint32_t *__restrict__ cand_rec, int slots, uint32_t *__restrict__ keys32, int64_t key_stride)
{
    __shared__ int32_t pt_lds[kSlots * kScoreWaves * kScorePagesPerWave];
    __shared__ __attribute__((aligned(16))) unsigned char stage_all[kScoreWaves * kScoreUnroll * kStagePage];
    __shared__ uint32_t ck_all[kScoreWaves * kLists * kSubStride];
    __shared__ __attribute__((aligned(16))) uint16_t samp[kHeadBlock * kSampStride];   // top 16 key bits
    __shared__ uint32_t lo_lds[kHeadBlock];
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[kHeadBlock * kHeadDim];
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int n = seq_lens[b];
    static_assert(kSlots >= 1 && kSlots <= 4, "1 to 4 slots per wave");
    const int tok0 = blockIdx.x * kSlots * kScoreTokensPerBlock;
    if (tok0 >= n) return;                                    // whole block exits together
    const int kk = min(min(k_per_seq[b], n), k_max);
    const int heads_here = min(kHeadBlock, group - hb * kHeadBlock);
    const int h0 = g * group + hb * kHeadBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    const bool head_lane = col < heads_here;                  // lanes of column col carry head col
    unsigned char *stage = stage_all + wave * kScoreUnroll * kStagePage;
    // Lane lists are interleaved entry by entry (entry e of list L at e * kLists + L), so
    // the 32 head lanes of an append, whatever their counts, write 32 different banks.
    uint32_t *ck = ck_all + wave * kLists * kSubStride;
    const int my_list = min(col, kHeadBlock - 1) * 4 + quad;   // this lane's list (head col, quad)

    const int pages_seq = (n + kPage - 1) / kPage;
    const int p_base = tok0 / kPage;                          // first page of this workgroup
    // slot s of this wave is the workgroup's slot 4 s + wave: pages p_begin .. p_end - 1
    auto slot_begin = [&](int sl) { return p_base + (sl * kScoreWaves + wave) * kScorePagesPerWave; };
    auto slot_end = [&](int sl) { return min(slot_begin(sl) + kScorePagesPerWave, pages_seq); };
    int p_begin = slot_begin(0), p_end = slot_end(0);
    const bool has_pages = p_begin < p_end;                   // wave-uniform
    {
        const int32_t *pt = page_table + (int64_t)b * max_pages;
        const int i = threadIdx.x;
#pragma unroll
        for (int j = i; j < kSlots * kScoreWaves * kScorePagesPerWave; j += kScoreWaves * 64)
            if (p_base + j < pages_seq) pt_lds[j] = pt[p_base + j];
        // the head block's q rows (16 B per thread), staged with the page slice
        if (i < heads_here * (kHeadDim / 8))
            *(u32x4 *)(q_lds + i * 8) = *(const u32x4 *)(q + ((int64_t)b * num_q_heads + h0) * kHeadDim + i * 8);
    }
    __syncthreads();                                          // page slice and q staged
    // MFMA B operand: lane (col, quad) holds head col's dims 32 s + 8 quad .. +7
    bf16x8 qb[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
        qb[s4] = head_lane ? *(const bf16x8 *)(q_lds + col * kHeadDim + 32 * s4 + 8 * quad)
                           : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

    const uint16_t *k_head = kc + (int64_t)g * kPage * kHeadDim;                 // + phys * Hkv * 4 KiB
    const int64_t page_elems = (int64_t)num_kv_heads * kPage * kHeadDim;
    // contiguous loads: chunk s (1 KiB) of a page, lane -> row 4 s + lane / 16, dims 8 (lane % 16)
    const int wr_off = (lane >> 4) * kStageRow + (lane & 15) * 16;
    // MFMA A operand: row col, dims 32 s + 8 quad -> bytes 64 s + 16 quad
    const int rd_off = col * kStageRow + quad * 16;
    uint32_t cnt = 0;                                         // entries of this lane's list so far
    uint32_t taken[kScorePagesPerWave * 4 / 32] = {0u, 0u, 0u, 0u};   // tokens this lane took
    uint32_t lo = 0xFFFFFFFFu;                                // head col's bound (set after the sample)
    float lo_f = __builtin_nanf("");                          // the smallest score whose key reaches lo

    // pages p, p + 1, clamped to pend - 1 (a group past the row re-reads a page of it)
    auto load_group = [&](u32x4 (&kr)[kScoreUnroll][4], int p, int pend) {
        int64_t phys[kScoreUnroll];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) phys[u] = pt_lds[min(p + u, pend - 1) - p_base];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const u32x4 *src = (const u32x4 *)(k_head + phys[u] * page_elems) + lane;
#pragma unroll
            for (int s = 0; s < 4; ++s) kr[u][s] = __builtin_nontemporal_load(src + 64 * s);
        }
    };
    // scores of page p + u of a staged group: lane holds tokens 4 quad .. +3 of head col
    auto stage_group = [&](const u32x4 (&kr)[kScoreUnroll][4]) {
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) *(u32x4 *)(stage + u * kStagePage + s * 4 * kStageRow + wr_off) = kr[u][s];
    };
    // MFMA A operands of staged page u, and the raw fp32 scores (as bits) they give:
    // lane holds tokens 4 quad .. +3 of head col
    auto read_operands = [&](int u, bf16x8 (&ka)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = *(const bf16x8 *)(stage + u * kStagePage + s * 64 + rd_off);
    };
    auto mfma_scores = [&](const bf16x8 (&ka)[4], uint32_t (&sc)[4]) {
        const f32x4 acc = score_mfma(ka, qb);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = __float_as_uint(acc[i]);
    };
    auto page_scores = [&](int u, uint32_t (&sc)[4]) {
        bf16x8 ka[4];
        read_operands(u, ka);
        mfma_scores(ka, sc);
    };
    // append the scores of page po of the wave (po = 0..31, a compile-time offset) whose
    // key reaches lo, i.e. score >= lo_f: every head lane keeps its own list of scores
    // (head col, tokens 4 quad .. +3 of each page), ascending by construction, and
    // marks the tokens it took in a 128-bit mask (bit 4 po + i); the flush recovers
    // each entry's token from the mask, merges the 4 lists of a head into token order
    // and turns scores into keys.  Inside the head lanes it is branch-free: every score
    // is written, a rejected one into the lane's own pad slot, which is never read.
    // (all-keys mode: every key goes to its head's key row; one buffer store per page,
    // dropped for the lanes that carry no head)
    const __amdgpu_buffer_rsrc_t key_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        keys32 + ((int64_t)b * num_q_heads + h0) * key_stride, 0, (int)(heads_here * key_stride * 4), kBufferDword3);
    auto append_page = [&](const uint32_t (&sc)[4], int po) {
        if constexpr (kAllKeys) {
            u32x4 kv;
#pragma unroll
            for (int i = 0; i < 4; ++i) kv[i] = score_key(__uint_as_float(sc[i]));
            const uint32_t off = (uint32_t)((col * key_stride + (p_begin + po) * kPage + 4 * quad) * 4);
            __builtin_amdgcn_raw_buffer_store_b128(kv, key_rsrc, head_lane ? off : kDropOffset, 0, 0);
            return;
        }
        if (!head_lane) return;
        const int t0 = (p_begin + po) * kPage + 4 * quad;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool take = (t0 + i < n) & (__uint_as_float(sc[i]) >= lo_f);
            const uint32_t at = (take & (cnt < (uint32_t)kSubCap)) ? cnt : (uint32_t)kSubCap;
            ck[at * kLists + my_list] = sc[i];
            taken[(4 * po + i) >> 5] |= (take ? 1u : 0u) << ((4 * po + i) & 31);
            cnt += take ? 1u : 0u;
        }
    };
    auto score_group = [&](u32x4 (&kr)[kScoreUnroll][4], int p, int p_next, int pend_next, bool reload) {
        stage_group(kr);
        sched_fence();
        if (reload) load_group(kr, p_next, pend_next);
        sched_fence();
        // the operands of every staged page first: LDS operations complete in order, so
        // an operand read issued after an append's writes would wait for them
        bf16x8 op[kScoreUnroll][4];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) read_operands(u, op[u]);
        sched_fence();
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            if (p + u < p_end) {                              // wave-uniform
                uint32_t sc[4];
                mfma_scores(op[u], sc);
                append_page(sc, p - p_begin + u);
            }
        }
        sched_fence();
    };
    // the sample: scores of the wave's first pages kept, their keys' top 16 bits to LDS
    // (0 for tokens past the row)
    uint32_t skey[kSamplePagesPerWave][4];
    auto sample_group = [&](u32x4 (&kr)[kScoreUnroll][4], int su0) {
        stage_group(kr);                                      // (a wave without pages stages
        sched_fence();                                        //  and loads its row's last page)
        load_group(kr, p_begin + su0 + kScoreBufs * kScoreUnroll, p_end);
        sched_fence();
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const int su = su0 + u, pp = p_begin + su;
            uint32_t sc[4] = {0u, 0u, 0u, 0u};
            if (pp < p_end) page_scores(u, sc);               // wave-uniform
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                skey[su][i] = sc[i];
                const int t = pp * kPage + 4 * quad + i;
                if (head_lane)
                    samp[col * kSampStride + (wave * kSamplePagesPerWave + su) * kPage + 4 * quad + i] =
                        (pp < p_end && t < n) ? (uint16_t)(score_key(__uint_as_float(sc[i])) >> 16) : (uint16_t)0;
            }
        }
        sched_fence();
    };

    // 1. the sample pages, with the next groups' loads in flight.  Group G of the wave
    //    (counted over its slots) lives in register buffer G mod kScoreBufs.
    u32x4 kb0[kScoreUnroll][4], kb1[kScoreUnroll][4], kb2[kScoreUnroll][4];
    auto buf = [&](auto G) -> u32x4 (&)[kScoreUnroll][4] {
        constexpr int i = decltype(G)::value % kScoreBufs;
        if constexpr (i == 0) return kb0;
        else if constexpr (i == 1) return kb1;
        else return kb2;
    };
    static_for<0, kScoreBufs>([&](auto G) {                   // unconditional: no control flow
        load_group(buf(G), p_begin + decltype(G)::value * kScoreUnroll, p_end);   // around loads in flight
        sched_fence();
    });
    if constexpr (!kAllKeys) {
    static_for<0, kSampleGroups>([&](auto G) { sample_group(buf(G), decltype(G)::value * kScoreUnroll); });
    lds_barrier();
    // 2. per head hh (one wave each): its bound, the r-th largest sample code found by bisection,
    //    r = mu + 6 sqrt(mu) + 8 for mu the expected number of samples at or above
    //    the k-th key (a bound above the k-th key sends the row to the slow path, so
    //    the margin keeps that below about 1e-9 per workgroup and head)
    for (int hh = wave; hh < heads_here; hh += kScoreWaves) {
        uint32_t b_lo = 0xFFFFFFFFu;                          // k' = 0 or N: no candidates needed
        if (kk > 0 && kk < n) {
            int s_valid = 0;
            for (int w = 0; w < kScoreWaves; ++w)
                s_valid += min(max(n - (p_base + w * kScorePagesPerWave) * kPage, 0), kSamplePagesPerWave * kPage);
            const float mu = (float)s_valid * (float)kk / (float)n;
            const uint32_t r = (uint32_t)ceilf(mu + 6.f * sqrtf(mu) + 8.f);
            b_lo = 0u;                                        // too few samples: keep everything
            if (r < (uint32_t)s_valid) {
                constexpr int per_lane = kBlockSample / 64;   // 16 codes
                uint32_t c[per_lane];
#pragma unroll
                for (int v = 0; v < per_lane / 8; ++v) {
                    const u32x4 w4 = *(const u32x4 *)&samp[hh * kSampStride + lane * per_lane + 8 * v];
                    c[8 * v + 0] = w4.x & 0xFFFFu; c[8 * v + 1] = w4.x >> 16;
                    c[8 * v + 2] = w4.y & 0xFFFFu; c[8 * v + 3] = w4.y >> 16;
                    c[8 * v + 4] = w4.z & 0xFFFFu; c[8 * v + 5] = w4.z >> 16;
                    c[8 * v + 6] = w4.w & 0xFFFFu; c[8 * v + 7] = w4.w >> 16;
                }
                uint32_t lo_c = 0, hi_c = 0x10000;            // count(code >= lo_c) >= r > count(code >= hi_c)
                while (hi_c - lo_c > 1) {
                    const uint32_t mid = (lo_c + hi_c) >> 1;
                    uint32_t m = 0;
#pragma unroll
                    for (int e = 0; e < per_lane; ++e) m += c[e] >= mid ? 1u : 0u;
                    if (wave_total(m) >= r) lo_c = mid; else hi_c = mid;
                }
                b_lo = lo_c << 16;
            }
        }
        if (lane == 0) lo_lds[hh] = b_lo;
    }
    lds_barrier();
    if (head_lane) lo = lo_lds[col];
    // lo = 0: every score; ~0: none (the comparison with a NaN is false)
    lo_f = lo == 0u ? -__builtin_inff() : __uint_as_float((lo & 0x80000000u) ? (lo & 0x7FFFFFFFu) : ~lo);
    // 3. the sample pages' candidates, then the rest of the stream
#pragma unroll
    for (int su = 0; su < kSamplePagesPerWave; ++su)
        if (p_begin + su < p_end) append_page(skey[su], su);
    }
    auto flush_slot = [&]() __attribute__((always_inline)) {
        if constexpr (kAllKeys) return;                       // the keys are already out
        // this wave's slot: per head one record (count, bound, largest key, then the
        // candidates in token order).  Head lane (col, quad) places its own entries:
        // the e-th set bit of its mask is the token of its e-th entry, which goes to
        // e + (entries of the head's other lanes with a lower token).  The records are
        // assembled in LDS (the stage tile takes the keys, this wave's quarter of the
        // sample codes the header and positions, both free now) and leave in whole
        // 128-byte lines: a partial line costs HBM a read-modify-write, and these
        // writes share the memory with the key stream.
        uint32_t *out_key = (uint32_t *)stage;                                 // [head][kCandCap]
        uint32_t *out_tail = (uint32_t *)(samp + wave * (kHeadBlock * kSampStride / kScoreWaves));
        static_assert(kHeadBlock * kCandCap * 4 <= kScoreUnroll * kStagePage, "keys fit the stage tile");
        static_assert(kHeadBlock * kRecTailWords * 4 <= kHeadBlock * kSampStride * 2 / kScoreWaves, "tails fit");
        static_assert(kHeadBlock * kSampStride * 2 / kScoreWaves % 16 == 0, "tails 16-byte aligned");
        wave_lds_sync();
        const int slot = p_begin / kScorePagesPerWave;
        uint32_t oc[4], om[4][4], total = 0;
        bool ovf = false;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            oc[q2] = (uint32_t)__shfl((int)cnt, col + 16 * q2, 64);
#pragma unroll
            for (int w = 0; w < 4; ++w) om[q2][w] = (uint32_t)__shfl((int)taken[w], col + 16 * q2, 64);
            ovf |= oc[q2] > (uint32_t)kSubCap;
            total += oc[q2];
        }
        uint32_t *tail = out_tail + min(col, kHeadBlock - 1) * kRecTailWords;
        uint16_t *tail_pos = (uint16_t *)(tail + 4);
        uint32_t kmax = 0;                                    // largest key this lane places
        if (head_lane && !ovf) {
            // the other lanes' entries in the mask words before word w (a prefix of
            // whole-word counts); inside word w only the partial word is counted
            uint32_t before_word[4], run = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                before_word[w] = run;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) run += q2 == quad ? 0u : (uint32_t)__popc(om[q2][w]);
            }
            uint32_t e = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t bits = taken[w];
                while (bits) {
                    const int j = 32 * w + __builtin_ctz(bits);       // 4 page + i
                    bits &= bits - 1u;
                    const int pg = j >> 2;
                    // other lanes' tokens below this one: their bits below 4 pg, and
                    // for the lower quads also their bits of page pg
                    const int b_lo = 4 * (pg & 7);
                    const uint32_t m_hi = (1u << b_lo) - 1u;                           // bits < 4 pg
                    const uint32_t m_lo = b_lo + 4 >= 32 ? 0xFFFFFFFFu : (1u << (b_lo + 4)) - 1u;
                    uint32_t f = e + before_word[w];
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2)
                        if (q2 != quad) f += (uint32_t)__popc(om[q2][w] & (q2 < quad ? m_lo : m_hi));
                    const uint32_t key = score_key(__uint_as_float(ck[e * kLists + my_list]));
                    kmax = max(kmax, key);
                    out_key[col * kCandCap + f] = key;
                    tail_pos[f] = (uint16_t)(pg * kPage + 4 * quad + (j & 3));
                    ++e;
                }
            }
        }
        // the slot's largest candidate key (bounds the select's radix digits)
        uint32_t hm = 0;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) hm = max(hm, (uint32_t)__shfl((int)kmax, col + 16 * q2, 64));
        if (head_lane && quad == 0) *(u32x4 *)tail = u32x4{ovf ? kCandOverflow : total, lo, hm, 0u};
        wave_lds_sync();
        // 16 B per lane: lanes 0..47 the key lines, lanes 0..31 the tail lines.  The
        // stores go through a buffer resource over the head's records, and a lane with
        // nothing to write aims past them, where the store is dropped: every wave issues
        // the same 2 kHeadBlock stores, so the compiler's waits for the next slot's
        // loads (issued before them) need not wait for the stores as well.
        const uint32_t row_bytes = (uint32_t)slots * kRecWords * 4u;
        const uint32_t at = (uint32_t)slot * kRecWords * 4u + 16u * lane;
#pragma unroll
        for (int hh = 0; hh < kHeadBlock; ++hh) {
            const uint32_t tot = (uint32_t)__shfl((int)(ovf ? 0u : total), hh, 64);
            const bool live = hh < heads_here;
            const int64_t row_h = (int64_t)b * num_q_heads + h0 + min(hh, heads_here - 1);
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc(cand_rec + row_h * slots * kRecWords, 0, (int)row_bytes, kBufferDword3);
            const int key_chunks = live ? (int)((tot + 31u) / 32u) * 8 : 0;                  // whole lines of keys
            const int tail_chunks = live ? (int)((4u + (tot + 1u) / 2u + 31u) / 32u) * 8 : 0; // header + positions
            const u32x4 kv = ((const u32x4 *)(out_key + hh * kCandCap))[min(lane, kCandCap / 4 - 1)];
            const u32x4 tv = ((const u32x4 *)(out_tail + hh * kRecTailWords))[min(lane, kRecTailWords / 4 - 1)];
            __builtin_amdgcn_raw_buffer_store_b128(kv, rsrc, lane < key_chunks ? at : kDropOffset, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(tv, rsrc, lane < tail_chunks ? at + kCandCap * 4 : kDropOffset, 0, 0);
        }
    };
    // the main phase of slot S: its pages after the sample (slot 0) or all of them,
    // fully unrolled: straight-line code lets the compiler wait for exactly the group it
    // stages, with the next groups in flight.  The last groups of a slot put the
    // next slot's first pages in flight, so the flush overlaps their loads.
    auto run_slot = [&](auto S) __attribute__((always_inline)) -> bool {
        constexpr int sl = decltype(S)::value;
        if constexpr (sl > 0) {
            p_begin = slot_begin(sl);
            p_end = slot_end(sl);
            if (p_begin >= p_end) return false;               // wave-uniform; later slots are empty too
            cnt = 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) taken[w] = 0u;
        }
        constexpr bool more = sl + 1 < kSlots;
        const int nb = more ? slot_begin(sl + 1) : 0, ne = more ? slot_end(sl + 1) : 0;
        static_for<sl == 0 && !kAllKeys ? kSampleGroups : 0, kSlotGroups>([&](auto GI) {
            constexpr int g = decltype(GI)::value;            // group in the slot
            constexpr int gn = g + kScoreBufs;                // the group its buffer loads next
            constexpr bool same = gn < kSlotGroups;
            score_group(buf(std::integral_constant<int, sl * kSlotGroups + g>{}), p_begin + g * kScoreUnroll,
                        same ? p_begin + gn * kScoreUnroll : nb + (gn - kSlotGroups) * kScoreUnroll,
                        same ? p_end : ne, same || more);
        });
        flush_slot();
        return true;
    };
    if (has_pages) {                                          // wave-uniform
        bool go = run_slot(std::integral_constant<int, 0>{});
        if constexpr (kSlots > 1) go = go && run_slot(std::integral_constant<int, 1>{});
        if constexpr (kSlots > 2) go = go && run_slot(std::integral_constant<int, 2>{});
        if constexpr (kSlots > 3) go = go && run_slot(std::integral_constant<int, 3>{});
        (void)go;
    }
}

// ---- 2. select ---------------------------------------------------------------------------

// Candidate keys and their in-slot positions gathered into LDS in token order.  The
// candidates of slot i are positions [first[i], first[i + 1]); blk[v / 64] is the
// slot of position 64 (v / 64), where the walk to position v's slot starts.
__device__ __forceinline__ int slot_of_position(const uint32_t *first, const uint32_t *blk, uint32_t v)
{
    int i = (int)blk[v >> 6];
    while (v >= first[i + 1]) ++i;
    return i;
}

struct LdsCandidates {
    const uint32_t *key, *first, *blk;
    const uint16_t *pos;                                      // token - slot start, per position
    __device__ int load8(int start, int n, uint32_t (&v)[8]) const { return load_keys8(key, start, n, v); }
    // tokens of positions start .. start + cnt - 1 (cnt <= 8, all below the total)
    __device__ void tokens8(int start, int cnt, int32_t (&t)[8]) const
    {
        int i = (int)blk[start >> 6];
        uint32_t f1 = first[i + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t v = (uint32_t)(start + e);
            if (e < cnt) {
                while (v >= f1) { ++i; f1 = first[i + 1]; }
            }
            t[e] = e < cnt ? i * kWaveTokens + pos[v] : -1;
        }
    }
};

// Generic path for one head: re-score every token to its full 32-bit key in the
// workspace row (from the K rows, or from the label rows for the lightweight
// indexer), then radix-select over the keys.  Called by the whole workgroup.
template <int kThreads>
__device__ __forceinline__ void select_rescore_generic(const SelectArgs &a, int64_t bh, int b, int h, int n, int kk,
                                                       uint32_t *hist, uint32_t *scratch, uint32_t *res,
                                                       int32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, quad = lane >> 4;
    const int g = h / a.group, hl = h - g * a.group, hb = hl / kHeadBlock, hn = hl - hb * kHeadBlock;
    const int heads_here = min(kHeadBlock, a.group - hb * kHeadBlock);
    uint32_t *krow = a.keys32 + bh * a.stride;
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages;
    if (a.labels) {                                           // lightweight indexer: label rows
        const int32_t *ch = a.channels + g * kLabelDims;
        const uint16_t *qrow = a.q + bh * kHeadDim;
        float qc[kLabelDims];
#pragma unroll
        for (int i = 0; i < kLabelDims; ++i) qc[i] = __uint_as_float((uint32_t)qrow[ch[i]] << 16);
        for (int tok = threadIdx.x; tok < n; tok += kThreads) {
            const int64_t row = ((int64_t)pt[tok >> 4] * a.num_kv_heads + g) * kPage + (tok & 15);
            const u32x4 *lr = (const u32x4 *)(a.labels + row * kLabelDims);
            krow[tok] = score_key(label_score(qc, lr[0], lr[1]));
        }
        __threadfence_block();
        __syncthreads();
        radix_select<kThreads>(RowKeys{krow}, n, kk, a.k_max, 0u, 32, 0u, hist, scratch, res, out);
        return;
    }
    bf16x8 qb[4];
    load_q_operand(qb, a.q, (int64_t)b * a.num_q_heads + g * a.group + hb * kHeadBlock, heads_here, col, quad);
    for (int t0 = wave * 16; t0 < n; t0 += (kThreads / 64) * 16) {
        const int tok = t0 + col;
        const int row = tok < n ? (pt[tok >> 4] * a.num_kv_heads + g) * kPage + (tok & 15) : -1;
        const f32x4 acc = rescore16(a.kc, row, qb, quad);
        if (col == hn) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + 4 * quad + i < n) krow[t0 + 4 * quad + i] = score_key(acc[i]);
        }
    }
    __threadfence_block();
    __syncthreads();
    radix_select<kThreads>(RowKeys{krow}, n, kk, a.k_max, 0u, 32, 0u, hist, scratch, res, out);
}

// grid (num_q_heads, batch); kThreads threads (512, or 1024 when the rows are fewer
// than the CUs); dynamic LDS holds the candidates.
template <int kThreads>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a)
{
    // keys[cap] | first[slots + 1] | blk[cap / 64] | positions (16-bit) [cap]
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ uint32_t scratch[kThreads / 64 + 2];
    __shared__ uint32_t res[8];
    __shared__ uint32_t blist[64];                            // keys of the threshold bin

    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * a.num_q_heads + h;
    const uint32_t *rec_row = a.cand_rec + bh * a.slots * kRecWords;
    // the first block of slot headers goes out before the row's length arrives
    u32x4 hdr0 = u32x4{0u, 0u, 0u, 0u};
    if (a.cap != 0 && (int)threadIdx.x < a.slots) hdr0 = *(const u32x4 *)(rec_row + threadIdx.x * kRecWords + kCandCap);
    const int n = a.seq_lens[b];
    int kk = min(min(a.k_per_seq[b], n), a.k_max);
    if (kk < 0) kk = 0;
    int32_t *out = a.idx_out + bh * a.k_max;
    if (kk == n || kk == 0) {                                 // everything, or nothing
        for (int i = threadIdx.x; i < a.k_max; i += kThreads) out[i] = i < kk ? i : -1;
        return;
    }
    if (a.all_keys) {
        radix_select<kThreads>(RowKeys{a.keys32 + bh * a.stride}, n, kk, a.k_max, 0u, 32, 0u, hist, scratch, res, out);
        return;
    }
    bool generic = a.cap == 0;
    uint32_t *ckey = dyn_lds, *first = dyn_lds + a.cap, *blk = first + a.slots + 1;
    uint16_t *cpos = (uint16_t *)(blk + (a.cap + 63) / 64);
    const int nslots = (n + kWaveTokens - 1) / kWaveTokens;
    uint32_t total = 0;
    if (threadIdx.x < 8) res[threadIdx.x] = 0u;
    if (!generic) {
        // 1. slot counts -> first[i], the place of slot i's first candidate.  An
        //    overflowed slot sends the row to the generic path.
        int bad = 0;
        uint32_t lo_max = 0u, hi_max = 0u;
        for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0u;
        for (int base = 0; base < a.slots; base += kThreads) {
            // loaded for every allocated slot (no wait for seq_lens), used below nslots
            const int i = base + (int)threadIdx.x;
            const bool in_ws = i < a.slots;
            const u32x4 hdr = base == 0 ? hdr0
                              : in_ws ? *(const u32x4 *)(rec_row + (int64_t)i * kRecWords + kCandCap)
                                      : u32x4{0u, 0u, 0u, 0u};
            const uint32_t c_raw = hdr.x, l = hdr.y, hv = hdr.z;
            uint32_t c = i < nslots ? c_raw : 0u;
            if (i < nslots) {
                lo_max = max(lo_max, l);
                if (c != 0u && c != kCandOverflow) hi_max = max(hi_max, hv);
            }
            const bool ovf = c == kCandOverflow;
            c = ovf ? 0u : c;
            bad |= __syncthreads_or(ovf ? 1 : 0);
            uint32_t tot;
            const uint32_t p0 = total + block_exclusive_scan<kThreads>(c, scratch, tot);
            if (in_ws) first[i] = p0;
            for (uint32_t v = (p0 + 63u) & ~63u; v < p0 + c && v < (uint32_t)a.cap; v += 64u) blk[v >> 6] = (uint32_t)i;
            total += tot;
        }
        if (threadIdx.x == 0) first[a.slots] = total;
        generic = bad != 0 || total < (uint32_t)kk || total > (uint32_t)a.cap;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            lo_max = max(lo_max, (uint32_t)__shfl_xor((int)lo_max, m, 64));
            hi_max = max(hi_max, (uint32_t)__shfl_xor((int)hi_max, m, 64));
        }
        if ((threadIdx.x & 63) == 0) {
            atomicMax(&res[6], lo_max);
            atomicMax(&res[7], hi_max);
        }
        __syncthreads();                                      // map, bounds and cleared histogram complete
    }
    if (generic) {
        select_rescore_generic<kThreads>(a, bh, b, h, n, kk, hist, scratch, res, out);
        return;
    }
    // 2. gather the candidates into LDS in token order: thread t takes list positions
    //    t, t + 512, ... (kGatherUnroll of them in flight at once), finds each one's
    //    slot, and loads its key and its 16-bit position from the slot's record; the
    //    first radix digit of d = key - lo is counted on the way.  lo is the largest
    //    bound: a key below it can never be selected (T must reach every bound), so
    //    such keys stay in place but take no part in the digits; a workgroup that kept
    //    all its tokens (bound 0, a row's short tail) then does not stretch the digits
    //    over the whole key range.  The largest candidate key gives the digits' span.
    const uint32_t lo = res[6], lo_max = lo, hi_max = res[7];
    const int bits = hi_max >= lo ? 32 - __clz((int)(hi_max - lo)) : 0;
    const int w0 = min(kHistBits, bits), sh0 = bits - w0;
    const uint32_t mask0 = (1u << w0) - 1u;
    uint32_t eligible = 0;                                    // keys >= lo this thread gathered
    for (uint32_t v0 = 0; v0 < total; v0 += kThreads * kGatherUnroll) {
        // every slot walk first, then every load, then their uses: a walk between two
        // loads would reuse registers that a load in flight still has to write, and the
        // load would be waited for before the next one goes out.  Positions past the
        // list re-read the last entry (in place, unused).
        const uint32_t *rec[kGatherUnroll];
        uint32_t jj[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const uint32_t v = min(v0 + u * kThreads + threadIdx.x, total - 1u);
            const int i = slot_of_position(first, blk, v);
            rec[u] = rec_row + (int64_t)i * kRecWords;
            jj[u] = v - first[i];
        }
        uint32_t key[kGatherUnroll], ps[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            key[u] = rec[u][jj[u]];
            ps[u] = ((const uint16_t *)(rec[u] + kCandCap + 4))[jj[u]];
        }
        asm volatile("" ::: "memory");                        // the loads stay above their uses
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const uint32_t v = v0 + u * kThreads + threadIdx.x;
            if (v < total) {
                ckey[v] = key[u];
                cpos[v] = ps[u];
                if (key[u] >= lo) {
                    ++eligible;
                    if (bits > 0) atomicAdd(&hist[((key[u] - lo) >> sh0) & mask0], 1u);
                }
            }
        }
    }
    eligible = wave_total(eligible);
    if ((threadIdx.x & 63) == 0) atomicAdd(&res[4], eligible);
    if (threadIdx.x == 0) { res[0] = 0u; res[1] = 0u; res[2] = 0u; }
    __syncthreads();
    if (res[4] < (uint32_t)kk) {                              // fewer than k keys reach every bound
        __syncthreads();
        select_rescore_generic<kThreads>(a, bh, b, h, n, kk, hist, scratch, res, out);
        return;
    }
    // 3. the k-th key T and r, the number of keys equal to T to take (the first ones):
    //    the first digit's bin b0 holds it; if the whole bin is taken and its floor
    //    already reaches every bound, the bin floor is T with all ties; otherwise the
    //    bin's few entries are ranked exactly by one wave.  The selection is valid if T
    //    reaches every workgroup bound.
    const LdsCandidates cands{ckey, first, blk, cpos};
    uint32_t T = lo, r = (uint32_t)kk;
    if (bits > 0) {
        threshold_bin_wave(hist, max(64, 1 << w0), (uint32_t)kk, res);
        const uint32_t b0 = res[0], need0 = (uint32_t)kk - res[1], floor0 = lo + (b0 << sh0);
        if (need0 == hist[b0] && floor0 >= lo_max) {
            T = floor0;
            r = 0xFFFFFFFFu;
        } else {
            for (uint32_t v = threadIdx.x; v < total; v += kThreads) {
                const uint32_t key = ckey[v];
                if (key >= lo && ((key - lo) >> sh0) == b0) {
                    const uint32_t at = atomicAdd(&res[2], 1u);
                    if (at < 64u) blist[at] = key;
                }
            }
            __syncthreads();
            const uint32_t m = res[2];
            if (m > 64u) {                                    // a crowded bin: full radix passes
                __syncthreads();
                if (!radix_select<kThreads>(cands, (int)total, kk, a.k_max, lo, bits, lo_max, hist, scratch, res, out))
                    select_rescore_generic<kThreads>(a, bh, b, h, n, kk, hist, scratch, res, out);
                return;
            }
            if (threadIdx.x < 64) {                           // need0-th largest of the bin, by rank
                const int lane = threadIdx.x;
                const uint32_t mine = lane < (int)m ? blist[lane] : 0u;
                uint32_t gt = 0, eq = 0;
                for (uint32_t j = 0; j < m; ++j) {
                    const uint32_t o = blist[j];
                    gt += o > mine ? 1u : 0u;
                    eq += o == mine ? 1u : 0u;
                }
                const uint64_t hit = __ballot(lane < (int)m && gt < need0 && need0 <= gt + eq);
                const int L = __ffsll((unsigned long long)hit) - 1;
                if (lane == L) { res[3] = mine; res[4] = need0 - gt; }
            }
            __syncthreads();
            T = res[3];
            r = res[4];
        }
    }
    if (T < lo_max) {                                         // some workgroup's bound lies above T
        __syncthreads();
        select_rescore_generic<kThreads>(a, bh, b, h, n, kk, hist, scratch, res, out);
        return;
    }
    compact_selected<kThreads>(cands, (int)total, kk, a.k_max, T, r, scratch, out);
}

// ---- host side ---------------------------------------------------------------------------

size_t index_topk_key_stride(int n_max) { return (size_t)((n_max + 127) / 128) * 128; }

int index_topk_slots(int n_max) { return (n_max + kWaveTokens - 1) / kWaveTokens; }

size_t index_topk_workspace_bytes(int batch, int num_q_heads, int n_max)
{
    // per (b, h): a 32-bit key row for the generic path, then per 512-token slot a
    // candidate record (count, bound, largest key, 32-bit keys, 16-bit positions)
    const size_t rows = (size_t)batch * num_q_heads, slots = (size_t)index_topk_slots(n_max);
    return rows * (index_topk_key_stride(n_max) * sizeof(uint32_t) + slots * kRecWords * sizeof(uint32_t));
}

SelectPlan plan_select(int k_max, int n_max, int slots)
{
    // LDS for the candidates.  A workgroup's bound is reached by about (n_w / 1024) r
    // of its n_w tokens, r = mu + 6 sqrt(mu) + 8 and mu = 1024 k / n, so a row has
    // about k + 6 sqrt(k n / 1024) + 8 n / 1024 candidates; the largest row bounds it
    // (15% margin).  Rows beyond the capacity take the re-scoring path.
    const double kd = k_max, nd = n_max;
    const double expect = kd + 6.0 * std::sqrt(kd * nd / 1024.0) + 8.0 * nd / 1024.0;
    // Beside the keys, the slot starts take (slots + 1) words, the walk starts one word
    // per 64 keys and the positions half a word per key.
    const int cap_lds = ((int)(kSelDynMax / sizeof(uint32_t)) - (slots + 3)) * 128 / 194;
    const int cap_want = (int)std::min<double>(1e9, std::ceil(1.15 * expect) + 256.0);
    int cap = std::max(0, std::min(std::min(cap_want, kSelCapMax), cap_lds));
    // A large k (or a row too long for the slot table) would overflow the slot lists or
    // the LDS: then the score pass writes every key to the key rows and the select
    // radix-selects over them (all-keys mode).  A slot expects r / 2 candidates, a
    // quarter of them in each 48-entry lane list; at 64 per slot (16 per list) even a
    // workgroup bound three deviations low leaves an overflow (a whole-row re-score)
    // more than six deviations away.  At k = N/8 on the 16 x 131072 sweep, 120 per slot
    // overflowed a few rows per hundred steps.
    const double mu = 1024.0 * kd / nd, r = mu + 6.0 * std::sqrt(mu) + 8.0;
    const bool all_keys = cap_want > cap || r / 2.0 > kSlotExpectMax;
    if (all_keys) cap = 0;
    const size_t dyn = cap == 0 ? 0
                                : (size_t)(cap + slots + 1 + (cap + 63) / 64) * sizeof(uint32_t) +
                                      (size_t)(cap + 1) / 2 * sizeof(uint32_t);
    return SelectPlan{cap, dyn, all_keys};
}

template <int kThreads>
static hipError_t launch_select_with(const SelectArgs &s, const SelectPlan &p, int batch, hipStream_t stream)
{
    if (p.dyn > 64 * 1024) {
        // raise the kernel's dynamic-LDS limit to the budget (a function attribute kept by
        // the runtime, not a stream operation; setting it again is harmless and keeps the
        // library free of state of its own)
        const hipError_t e = hipFuncSetAttribute((const void *)select_kernel<kThreads>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kSelDynMax);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(select_kernel<kThreads>, dim3(s.num_q_heads, batch), dim3(kThreads), p.dyn, stream, s);
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &s, const SelectPlan &p, int batch, hipStream_t stream)
{
    // Fewer rows than CUs leave CUs idle: long rows then take twice the threads (the
    // 160-row long-retrieval batch measured 3.6 us faster; with a row or more per CU,
    // or short rows, 512 threads measured faster).
    const bool few_rows = (int64_t)s.num_q_heads * batch < kCUs;
    const bool long_rows = s.cap >= 4096 || (s.all_keys && s.stride >= 65536);
    if (few_rows && long_rows) return launch_select_with<1024>(s, p, batch, stream);
    return launch_select_with<kSelThreads>(s, p, batch, stream);
}

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int head_blocks = (group + kHeadBlock - 1) / kHeadBlock;
    const int64_t stride = (int64_t)index_topk_key_stride(a.n_max);
    const int slots = index_topk_slots(a.n_max);
    const size_t rows = (size_t)a.batch * a.num_q_heads;
    uint32_t *keys32 = (uint32_t *)a.ws;
    uint32_t *cand_rec = keys32 + rows * stride;              // 512 B multiple: records start on lines
    const SelectPlan plan = plan_select(a.k_max, a.n_max, slots);

    // Two slots per wave when that gives every CU two workgroups for at most two rounds:
    // a workgroup's first flush then overlaps its second half's loads, and half as many
    // workgroups wait for their last stores.  Longer grids (many rounds of ragged rows)
    // measured faster with one slot.
    const int64_t blocks2 = (int64_t)((a.n_max + 2 * kScoreTokensPerBlock - 1) / (2 * kScoreTokensPerBlock)) *
                            a.num_kv_heads * head_blocks * a.batch;
    const bool two = blocks2 >= 2 * kCUs && blocks2 <= 4 * kCUs;
    const int per_block = (two ? 2 : 1) * kScoreTokensPerBlock;
    const dim3 sgrid((a.n_max + per_block - 1) / per_block, a.num_kv_heads * head_blocks, a.batch);
    auto launch_score = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, sgrid, dim3(kScoreWaves * 64), 0, stream, (const uint16_t *)a.k_cache,
                           a.page_table, a.seq_lens, (const uint16_t *)a.q, a.k_per_seq, a.num_q_heads,
                           a.num_kv_heads, group, head_blocks, a.max_pages, a.k_max, cand_rec, slots, keys32,
                           stride);
    };
    if (plan.all_keys) {
        if (two) launch_score(score_kernel<2, true>);
        else launch_score(score_kernel<1, true>);
    } else {
        if (two) launch_score(score_kernel<2, false>);
        else launch_score(score_kernel<1, false>);
    }
    SelectArgs s{(const uint16_t *)a.k_cache, a.page_table, a.seq_lens, a.k_per_seq, (const uint16_t *)a.q,
                 cand_rec, slots, plan.cap, plan.all_keys ? 1 : 0, keys32, stride, a.num_q_heads, a.num_kv_heads,
                 group, a.max_pages, a.k_max, a.idx_out, nullptr, nullptr};
    return launch_select(s, plan, a.batch, stream);
}

}  // namespace sdi
