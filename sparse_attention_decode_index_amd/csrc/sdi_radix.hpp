// Exact radix selection over 32-bit keys for one (b, q head) row per workgroup
// (gfx950): histogram-threshold search by one wave, radix passes over key
// digits, and an ordered compaction that writes the selected positions
// ascending.  Shared by the token indexer and the page selection.
#pragma once

#include "sdi_device.hpp"

namespace sdi {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPerThread = 8;
constexpr int kSelTile = kSelThreads * kSelPerThread;

// Largest bin B of hist[0..nbins) (nbins = 64 * per, per <= 64) with
// sum_{bins >= B} >= need, found by one wave in two parallel levels: lane l sums
// bins top - l*per ... (from the highest bins down; hist 16-byte aligned when
// per >= 4), a wave scan locates the lane
// group holding the crossing, and a second scan over that group's `per` bins
// locates the bin.  Every lane of the calling wave gets bin and above (the count
// over bins > B).  Returns false (outputs untouched) if the total is below need.
__device__ __forceinline__ bool wave_threshold(const uint32_t *hist, int nbins, uint32_t need, uint32_t &bin,
                                               uint32_t &above)
{
    const int lane = threadIdx.x & 63, per = nbins / 64;
    const int top = nbins - 1 - lane * per;
    uint32_t mine = 0;
    if (per >= 4) {                                           // this lane's bins, 16-byte aligned
        const u32x4 *h4 = (const u32x4 *)(hist + (top - per + 1));
#pragma unroll 16
        for (int i = 0; i < per / 4; ++i) {
            const u32x4 v = h4[i];
            mine += v.x + v.y + v.z + v.w;
        }
    } else {
        for (int i = 0; i < per; ++i) mine += hist[top - i];
    }
    const uint32_t x = wave_inclusive_scan(mine);
    const uint64_t cross = __ballot(x >= need);
    if (cross == 0) return false;
    const int L = __ffsll((unsigned long long)cross) - 1;
    const uint32_t before = __shfl(x - mine, L, 64);
    const int top_l = nbins - 1 - L * per;
    const uint32_t c = lane < per ? hist[top_l - lane] : 0u;
    const uint32_t y = before + wave_inclusive_scan(c);
    const uint64_t cross2 = __ballot(lane < per && y >= need);
    const int I = __ffsll((unsigned long long)cross2) - 1;
    bin = (uint32_t)(top_l - I);
    above = __shfl(y - c, I, 64);
    return true;
}

// Sum of v over the 64 lanes of the wave, in every lane.
__device__ __forceinline__ uint32_t wave_total(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(v), 63);
}

// Workgroup form: wave 0 searches, res[0] = bin, res[1] = above; ends with a barrier.
__device__ __forceinline__ void threshold_bin_wave(const uint32_t *hist, int nbins, uint32_t need, uint32_t *res)
{
    if (threadIdx.x < 64) {
        uint32_t bin, above;
        if (wave_threshold(hist, nbins, need, bin, above) && threadIdx.x == 0) { res[0] = bin; res[1] = above; }
    }
    __syncthreads();
}

// Keys [start, start + 8) of a 32-bit key row, clipped to n.
__device__ __forceinline__ int load_keys8(const uint32_t *src, int start, int n, uint32_t (&v)[8])
{
    if (start + 8 <= n) {
        const u32x4 a = *(const u32x4 *)(src + start), c = *(const u32x4 *)(src + start + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        return 8;
    }
    const int cnt = n > start ? n - start : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < cnt ? src[start + e] : 0u;
    return cnt;
}

// A full 32-bit key row in the workspace: position = token.
struct RowKeys {
    const uint32_t *key;
    __device__ int load8(int start, int n, uint32_t (&v)[8]) const { return load_keys8(key, start, n, v); }
    __device__ void tokens8(int start, int cnt, int32_t (&t)[8]) const
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = start + e;
    }
};

template <int kThreads = kSelThreads, class Src>
__device__ __forceinline__ void compact_selected(const Src &src, int n, int kk, int k_max, uint32_t T, uint32_t r,
                                                 uint32_t *scratch, int32_t *__restrict__ out);

// Exact selection over n keys in token order, every key >= base: radix passes over
// the digits of d = key - base (d < 2^bits), kHistBits at a time from the top, find
// the kk-th largest key T and how many keys equal to T to take (the first ones,
// i.e. the lowest tokens); one ordered-compaction pass then writes the selected
// tokens ascending and pads the row with -1.  Returns false, writing nothing, if
// T < min_t.  With first_hist_ready the caller has already counted the first digit
// into hist (and zeroed res[0..1]).
template <int kThreads = kSelThreads, class Src>
__device__ __forceinline__ bool radix_select(const Src &src, int n, int kk, int k_max, uint32_t base, int bits,
                                             uint32_t min_t, uint32_t *hist, uint32_t *scratch, uint32_t *res,
                                             int32_t *__restrict__ out, bool first_hist_ready = false)
{
    uint32_t prefix = 0, need = (uint32_t)kk;
    int hi = bits;                                           // digits above bit hi are fixed (= prefix)
    bool ready = first_hist_ready;                           // the caller built the first digit's histogram
#pragma unroll 1
    while (hi > 0) {
        const int w = min(kHistBits, hi), lo = hi - w, nb = max(64, 1 << w);
        if (!ready) {
            for (int i = threadIdx.x; i < nb; i += kThreads) hist[i] = 0u;
            if (threadIdx.x == 0) { res[0] = 0u; res[1] = 0u; }
            __syncthreads();
            for (int i0 = 0; i0 < n; i0 += kThreads * kSelPerThread) {
                uint32_t v[8];
                const int cnt = src.load8(i0 + threadIdx.x * kSelPerThread, n, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t d = v[e] - base;
                    if (e < cnt && v[e] >= base && (hi == 32 || (d >> hi) == prefix))
                        atomicAdd(&hist[(d >> lo) & ((1u << w) - 1u)], 1u);
                }
            }
            __syncthreads();
        }
        ready = false;
        threshold_bin_wave(hist, nb, need, res);
        need -= res[1];
        prefix = (prefix << w) | res[0];
        hi = lo;
        __syncthreads();                                     // res consumed before its next write
    }
    prefix += base;
    const uint32_t T = prefix, r = need;                     // take keys > T and the first r keys == T
    if (T < min_t) return false;
    compact_selected<kThreads>(src, n, kk, k_max, T, r, scratch, out);
    return true;
}

// Ordered compaction: writes, in token order, the keys > T and the first r keys == T
// (at most kk tokens), then pads the row to k_max with -1.
template <int kThreads, class Src>
__device__ __forceinline__ void compact_selected(const Src &src, int n, int kk, int k_max, uint32_t T, uint32_t r,
                                                 uint32_t *scratch, int32_t *__restrict__ out)
{
    constexpr int kTile = kThreads * kSelPerThread;
    uint32_t run_sel = 0, run_eq = 0;
    for (int base = 0; base < n; base += kTile) {
        uint32_t v[8];
        const int start = base + threadIdx.x * kSelPerThread;
        const int cnt = src.load8(start, n, v);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gt += (e < cnt && v[e] > T) ? 1u : 0u;
            eq += (e < cnt && v[e] == T) ? 1u : 0u;
        }
        int32_t tk[8];
        if (gt + eq > 0u) src.tokens8(start, cnt, tk);        // loads in flight before the scan
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan<kThreads>((eq << 16) | gt, scratch, tot);
        const uint32_t eq_left = r > run_eq ? r - run_eq : 0u;
        uint32_t pos = run_sel + (pre & 0xFFFFu) + min(pre >> 16, eq_left);
        uint32_t eq_rank = run_eq + (pre >> 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e < cnt) {
                bool take = v[e] > T;
                if (v[e] == T) take = (eq_rank++ < r);
                if (take) {
                    if (pos < (uint32_t)kk) out[pos] = tk[e];
                    ++pos;
                }
            }
        }
        run_sel += (tot & 0xFFFFu) + min(tot >> 16, eq_left);
        run_eq += tot >> 16;
    }
    for (int i = (int)run_sel + threadIdx.x; i < k_max; i += kThreads) out[i] = -1;
}

}  // namespace sdi
