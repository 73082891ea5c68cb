// Shared layout of the top-k indexers (gfx950): candidate slots and their records in
// the index workspace, the select kernel's arguments and launch plan.  The exact
// indexer (full K rows) and the lightweight one (reduced-channel label rows) both
// write these records and both use select_kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sdi_device.hpp"

namespace sdi {

constexpr int kHeadBlock = 8;                                 // query heads scored per workgroup
constexpr int kCUs = 256;                                     // MI355X compute units
constexpr int kScoreWaves = 4;                                // waves per score workgroup
constexpr int kScorePagesPerWave = 32;
constexpr int kWaveTokens = kScorePagesPerWave * kPage;       // 512 tokens: one candidate slot
constexpr int kScoreTokensPerBlock = kScoreWaves * kWaveTokens;
constexpr int kLabelDims = 16;                                // channels of a label row
constexpr int kCandCap = 192;                                 // candidates kept per (slot, head)
constexpr uint32_t kCandOverflow = 0xFFFFFFFFu;               // slot count of an overflowed list
constexpr double kSlotExpectMax = 64.0;                       // larger expected slot counts: all-keys mode
// A slot's record for one head, 1280 B (ten 128-byte lines): 32-bit keys [0, 192),
// then the tail: count, bound, largest key, 0, and the 16-bit positions (token - slot
// start) in token order.
constexpr int kRecTailWords = 128;                            // 512 B: 4 header words + 192 positions
constexpr int kRecWords = kCandCap + kRecTailWords;
// Buffer resource word 3 for untyped 32-bit accesses on gfx9, and an offset past any
// row of records (a buffer store there is dropped by the range check).
constexpr int kBufferDword3 = 0x00020000;
constexpr uint32_t kDropOffset = 0x80000000u;
static_assert(4 + kCandCap / 2 <= kRecTailWords && kRecWords * 4 % 128 == 0, "record layout");
constexpr int kSelCapMax = 32768;                             // candidates gathered into LDS
constexpr int kSelDynMax = 136 * 1024;                        // dynamic LDS: candidate keys + slot starts


struct SelectArgs {
    const uint16_t *kc;
    const int32_t *page_table, *seq_lens, *k_per_seq;
    const uint16_t *q;
    const uint32_t *cand_rec;                                 // [row][slot] records of kRecWords
    int slots;                                                // slots per row
    int cap;                                                  // candidates the LDS holds (0: generic only)
    int all_keys;                                             // the score pass wrote every key to keys32
    uint32_t *keys32;                                         // generic-path scratch, one row per (b, h)
    int64_t stride;
    int num_q_heads, num_kv_heads, group, max_pages, k_max;
    int32_t *idx_out;
    const uint16_t *labels;                                   // lightweight indexer: label rows (else NULL)
    const int32_t *channels;                                  // ... and their channel lists [Hkv][kLabelDims]
};

// Reduced-channel score of one label row (16 bf16, two 16-byte words) against the
// query's values on those channels: an fp32 multiply-add chain over channel order
// 0..15, shared by the label score pass and the select's re-scoring path so both
// produce the same keys.
__device__ __forceinline__ float label_score(const float (&qc)[kLabelDims], const u32x4 &w0, const u32x4 &w1)
{
    float l[kLabelDims];
    unpack8(w0, l);
    unpack8(w1, l + 8);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kLabelDims; ++i) s = fmaf(qc[i], l[i], s);
    return s;
}

// The select launch: LDS capacity for the candidates and whether the score pass
// writes every key instead (all-keys mode).
struct SelectPlan {
    int cap;
    size_t dyn;
    bool all_keys;
};
SelectPlan plan_select(int k_max, int n_max, int slots);
hipError_t launch_select(const SelectArgs &s, const SelectPlan &p, int batch, hipStream_t stream);
// the index workspace: a 32-bit key row per (b, q head), then the slot records
int index_topk_slots(int n_max);

}  // namespace sdi
