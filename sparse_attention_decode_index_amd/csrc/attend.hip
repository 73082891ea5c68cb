// Sparse gather-attend for the context-sparse decode step (gfx950).
//
// The sparse decode mode of the context-sparsity paper (Fig. 1a) reads only the
// k selected K/V rows of each (sequence, query head); the selections differ per
// token, per query and per head (paper section 1), so each query head gathers its
// own rows and there is no shared contraction for MFMA: this is a matrix-vector
// product on the vector ALU.  Softmax over the selected rows uses the running
// (max, sum, accumulator) merge of FlashAttention's tiling (survey page, section
// 5.1) in fp32, split over chunks of the index list, and the chunk partials are
// combined by merge_kernel with a log-sum-exp merge.
//
// Work decomposition: a workgroup of W waves takes 64 W consecutive entries of one
// (b, h) index row, 64 per wave.  Rows of up to 1024 entries take one workgroup
// (W = ceil(k_max / 64)) and need no second launch; longer rows are cut into chunks
// of 4 waves whose partials merge_kernel combines.  Inside a wave, each group of 16
// lanes owns one gathered row at a time (16 lanes x 16 B = the 256 B row, one
// 128-bit load per lane for K and one for V); 8 (wide workgroups) or all 16 (chunks)
// rows of a group are in flight at once, and each group keeps its own running
// softmax state; the 4 groups, then the W waves, are merged at the end.
//
// Two-list mode (stochastic selection): row (b, h) lists its first k'_b = min(k_b,
// k_max) top-k entries followed by its first s'_b = min(s_b, s_max) drawn entries, and
// every drawn entry carries the row's weight w (the number of residual tokens each
// draw stands for).  The weight enters as log2(w) added to the entry's base-2 logit,
// so w e^{l} is what the softmax sums see.  Chunks past k'_b + s'_b do no work and
// are not merged, as chunks past k'_b are in the one-list mode.
#include "sdi_device.hpp"
#include "sdi_launch.hpp"
#include "../../include/sparse_decode.h"

#include <mutex>

namespace sdi {

constexpr int kAttMaxWaves = 16;
constexpr int kAttPerWave = 64;
constexpr int kAttWideMax = kAttMaxWaves * kAttPerWave; // rows up to 1024 entries: one workgroup each
constexpr int kAttChunkWaves = 4;                       // longer rows: 256-entry chunks + a merge

// Rows of up to 1024 entries get one workgroup of ceil(k_max / 64) waves that writes
// the output itself.  Longer (or ragged) rows are cut into 256-entry chunks of 4
// waves: small workgroups keep a CU busy when a row's last chunk is short, and a
// wave's 16 rows per lane group are all in flight at once.
int attend_waves(int k_max)
{
    return k_max <= kAttWideMax ? (k_max + kAttPerWave - 1) / kAttPerWave : kAttChunkWaves;
}
constexpr float kLog2e = 1.4426950408889634f;

// grid (splits, num_q_heads, batch); 64 W threads, W <= MAXW; BATCH rows per 16-lane
// group are loaded at once (16 = all of them).  SAMPLED: two-list mode.
template <int MAXW, int BATCH, bool SAMPLED>
__global__ __launch_bounds__(MAXW * 64) void attend_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ k_per_seq, int num_q_heads, int num_kv_heads, int group, int max_pages, int k_max,
    float scale_log2, int splits, float *__restrict__ part_ml, float *__restrict__ part_acc,
    float *__restrict__ out, const int32_t *__restrict__ sample, const float *__restrict__ sample_weight,
    const int32_t *__restrict__ s_per_seq, int s_max)
{
    __shared__ float red_acc[MAXW][kHeadDim];
    __shared__ float red_ml[MAXW][2];
    const int waves = blockDim.x >> 6;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const int g = h / group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, sub = lane & 15;
    const int i0 = split * waves * kAttPerWave;
    const int i = i0 + wave * kAttPerWave + lane;   // the entry this lane resolves
    // The lane's index entry and the q row load together with the row's counts (the
    // entry is clamped into the row and discarded below when i >= k'), so the index
    // load does not wait for k_per_seq.  Absent per-sequence counts read seq_lens in
    // their place (value unused): no load sits behind a branch on a null pointer.
    const int n = seq_lens[b];
    const int k_raw = (k_per_seq ? k_per_seq : seq_lens)[b];
    const int s_raw = SAMPLED ? (s_per_seq ? s_per_seq : seq_lens)[b] : 0;
    const int j_top = idx[bh * k_max + min(i, k_max - 1)];
    const u32x4 qw = *(const u32x4 *)(q + bh * kHeadDim + sub * 8);
    int kk = k_per_seq ? min(k_raw, k_max) : k_max;
    if (kk < 0) kk = 0;
    int len = kk;                            // entries of this row
    if (SAMPLED) len += max(s_per_seq ? min(s_raw, s_max) : s_max, 0);
    // A chunk past the row's entries exits.  The one-workgroup form (split 0 only) has no
    // such branch: with nothing listed every row is masked and it writes zeros below, and
    // without the branch the index and q loads above are issued before the counts arrive.
    if (MAXW != kAttMaxWaves && i0 >= len) {
        if (splits == 1)
            for (int t = threadIdx.x; t < kHeadDim; t += blockDim.x) out[bh * kHeadDim + t] = 0.f;
        return;                              // (chunks past k are never merged)
    }

    float qf[8];
    unpack8(qw, qf);
#pragma unroll
    for (int d = 0; d < 8; ++d) qf[d] *= scale_log2;

    // Each lane resolves one index of the wave's 64 to a cache row number (-1 = skip);
    // in two-list mode also to its base-2 log weight (0 for top-k entries).
    int my_row = -1;
    float my_lw = 0.f;
    {
        int j = -1;
        if (i < kk) {
            j = j_top;
        } else if (SAMPLED && i < len) {
            j = sample[bh * s_max + (i - kk)];
            my_lw = log2f(sample_weight[bh]);
        }
        if (j >= 0 && j < n) {
            const int page = page_table[(int64_t)b * max_pages + (j >> 4)];
            my_row = (page * num_kv_heads + g) * kPage + (j & 15);
        }
    }

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.f;

#pragma unroll
    for (int r0 = 0; r0 < kAttPerWave / 4; r0 += BATCH) {
        u32x4 kw[BATCH], vw[BATCH];
        int rows[BATCH];
        float lws[BATCH];
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            rows[r] = __shfl(my_row, (r0 + r) * 4 + grp, 64);
            lws[r] = SAMPLED ? __shfl(my_lw, (r0 + r) * 4 + grp, 64) : 0.f;
            kw[r] = u32x4{0u, 0u, 0u, 0u};
            vw[r] = u32x4{0u, 0u, 0u, 0u};
            if (rows[r] >= 0) {
                const int64_t off = (int64_t)rows[r] * kHeadDim + sub * 8;
                kw[r] = __builtin_nontemporal_load((const u32x4 *)(kc + off));
                vw[r] = __builtin_nontemporal_load((const u32x4 *)(vc + off));
            }
        }
        float x[BATCH];
        float bmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            float kf[8];
            unpack8(kw[r], kf);
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < 8; ++d) s = fmaf(qf[d], kf[d], s);
            s = row16_sum(s);
            x[r] = rows[r] >= 0 ? (SAMPLED ? s + lws[r] : s) : -INFINITY;
            bmax = fmaxf(bmax, x[r]);
        }
        const float m_new = fmaxf(m, bmax);
        if (m_new != -INFINITY) {
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[d] *= alpha;
#pragma unroll
            for (int r = 0; r < BATCH; ++r) {
                const float p = fast_exp2(x[r] - m_new);
                float vf[8];
                unpack8(vw[r], vf);
                l += p;
#pragma unroll
                for (int d = 0; d < 8; ++d) acc[d] = fmaf(p, vf[d], acc[d]);
            }
            m = m_new;
        }
    }

    // Merge the 4 groups of this wave (lanes xor 16 and xor 32 hold the same dims).
    float M = fmaxf(m, __shfl_xor(m, 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(m - M);
    l *= f;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        float a = acc[d] * f;
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
        acc[d] = a;
    }
    if (grp == 0) {
#pragma unroll
        for (int d = 0; d < 8; ++d) red_acc[wave][sub * 8 + d] = acc[d];
        if (sub == 0) { red_ml[wave][0] = M; red_ml[wave][1] = l; }
    }
    __syncthreads();

    // Merge the waves; thread t owns output dims t, t + blockDim.x, ... (one wave has 64 threads).
    for (int t = threadIdx.x; t < kHeadDim; t += blockDim.x) {
        float Mw = red_ml[0][0];
        for (int w = 1; w < waves; ++w) Mw = fmaxf(Mw, red_ml[w][0]);
        float L = 0.f, A = 0.f;
        for (int w = 0; w < waves; ++w) {
            const float fw = (Mw == -INFINITY) ? 0.f : fast_exp2(red_ml[w][0] - Mw);
            L += fw * red_ml[w][1];
            A += fw * red_acc[w][t];
        }
        if (splits == 1) {
            out[bh * kHeadDim + t] = L > 0.f ? A / L : 0.f;
        } else {
            const int64_t ps = bh * splits + split;
            part_acc[ps * kHeadDim + t] = A;
            if (t == 0) { part_ml[ps * 2] = Mw; part_ml[ps * 2 + 1] = L; }
        }
    }
}

// Log-sum-exp merge of per-chunk partials (m, l, acc[128]) of each (b, h).
// live chunks = ceil(count / per_chunk) with count = min(k_b, k_max) (sparse), N_b
// (dense), or min(k_b, k_max) + min(s_b, s_max) (two-list mode: counts2 = s_b).  grid (num_q_heads, batch); 512 threads: the chunk weights
// e^{m_s - M} are computed once into LDS, then 4 groups of 128 threads (one dim
// each) sum over interleaved chunks and combine their sums in LDS.
constexpr int kMergeThreads = 512;
constexpr int kMergeGroups = kMergeThreads / kHeadDim;
constexpr int kMergeWeights = 4096;                       // chunk weights kept in LDS

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *__restrict__ part_ml,
                                                              const float *__restrict__ part_acc, int splits,
                                                              int per_chunk, const int32_t *__restrict__ counts,
                                                              int count_cap, const int32_t *__restrict__ counts2,
                                                              int count_cap2, int num_q_heads, float *__restrict__ out)
{
    __shared__ float wts[kMergeWeights];
    __shared__ float red[kMergeThreads / 64];
    __shared__ float gsum[kMergeGroups][kHeadDim];
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    int cnt = counts ? min(counts[b], count_cap) : count_cap;
    if (cnt < 0) cnt = 0;
    if (count_cap2 > 0) cnt += max(counts2 ? min(counts2[b], count_cap2) : count_cap2, 0);
    const int live = min(splits, (cnt + per_chunk - 1) / per_chunk);
    const float *ml = part_ml + bh * splits * 2;

    // M = max of the chunk maxima
    float m = -INFINITY;
    for (int s = t; s < live; s += kMergeThreads) m = fmaxf(m, ml[2 * s]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);
    __syncthreads();

    // weights and L = sum_s e^{m_s - M} l_s
    float l = 0.f;
    for (int s = t; s < live; s += kMergeThreads) {
        const float f = (M == -INFINITY) ? 0.f : fast_exp2(ml[2 * s] - M);
        if (s < kMergeWeights) wts[s] = f;
        l += f * ml[2 * s + 1];
    }
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; ++w) L += red[w];

    // accumulators: group j sums chunks j, j + 4, ...
    const int d = t % kHeadDim, grp = t / kHeadDim;
    const float *pa = part_acc + bh * splits * kHeadDim + d;
    float A = 0.f;
    for (int s = grp; s < live; s += kMergeGroups) {
        const float f = s < kMergeWeights ? wts[s] : ((M == -INFINITY) ? 0.f : fast_exp2(ml[2 * s] - M));
        A = fmaf(f, pa[(int64_t)s * kHeadDim], A);
    }
    gsum[grp][d] = A;
    __syncthreads();
    if (t < kHeadDim) {
        float tot = 0.f;
#pragma unroll
        for (int j = 0; j < kMergeGroups; ++j) tot += gsum[j][t];
        out[bh * kHeadDim + t] = L > 0.f ? tot / L : 0.f;
    }
}

int attend_splits(int k_max)
{
    const int per_block = attend_waves(k_max) * kAttPerWave;
    return (k_max + per_block - 1) / per_block;
}

size_t attend_workspace_bytes(int batch, int num_q_heads, int k_max)
{
    const int splits = attend_splits(k_max);
    if (splits <= 1) return 0;
    return (size_t)batch * num_q_heads * splits * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_merge(const float *part_ml, const float *part_acc, int splits, int per_chunk,
                        const int32_t *counts, int count_cap, int batch, int num_q_heads, float *out,
                        hipStream_t stream, const int32_t *counts2, int count_cap2)
{
    hipLaunchKernelGGL(merge_kernel, dim3(num_q_heads, batch), dim3(kMergeThreads), 0, stream, part_ml, part_acc,
                       splits, per_chunk, counts, count_cap, counts2, count_cap2, num_q_heads, out);
    return hipGetLastError();
}

template <bool SAMPLED>
static hipError_t launch_attend_mode(const AttendArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int total = SAMPLED ? a.k_max + a.s_max : a.k_max;   // entries of a row
    const int splits = attend_splits(total);
    const size_t bhs = (size_t)a.batch * a.num_q_heads * splits;
    float *part_acc = (float *)a.ws;
    float *part_ml = splits > 1 ? part_acc + bhs * kHeadDim : nullptr;
    const int waves = attend_waves(total);
    const dim3 grid(splits, a.num_q_heads, a.batch);
    if (total <= kAttWideMax)
        hipLaunchKernelGGL((attend_kernel<kAttMaxWaves, 8, SAMPLED>), grid, dim3(waves * 64), 0, stream,
                           (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.page_table, a.seq_lens,
                           (const uint16_t *)a.q, a.idx, a.k_per_seq, a.num_q_heads, a.num_kv_heads, group,
                           a.max_pages, a.k_max, a.scale * kLog2e, splits, part_ml, part_acc, a.out, a.sample,
                           a.sample_weight, a.s_per_seq, a.s_max);
    else
        hipLaunchKernelGGL((attend_kernel<kAttChunkWaves, 16, SAMPLED>), grid, dim3(waves * 64), 0, stream,
                           (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.page_table, a.seq_lens,
                           (const uint16_t *)a.q, a.idx, a.k_per_seq, a.num_q_heads, a.num_kv_heads, group,
                           a.max_pages, a.k_max, a.scale * kLog2e, splits, part_ml, part_acc, a.out, a.sample,
                           a.sample_weight, a.s_per_seq, a.s_max);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    return launch_merge(part_ml, part_acc, splits, waves * kAttPerWave, a.k_per_seq, a.k_max, a.batch,
                        a.num_q_heads, a.out, stream, SAMPLED ? a.s_per_seq : nullptr, SAMPLED ? a.s_max : 0);
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t stream)
{
    return a.sample ? launch_attend_mode<true>(a, stream) : launch_attend_mode<false>(a, stream);
}

// ---- allocation-free form ----------------------------------------------------------------
// For callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops): the chunk partials of rows longer than one workgroup go to one fixed
// device array per GPU instead of a caller workspace.  Each call writes the partials it
// merges before merge_kernel reads them, so nothing in the array has to start at zero;
// calls that overlap on one GPU share the array and race.
constexpr size_t kNoAllocBytes = (size_t)32 << 20;                      // 32 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];                                   // its device address, per GPU

int launch_attend_noalloc(AttendArgs a, hipStream_t stream)
{
    if (attend_workspace_bytes(a.batch, a.num_q_heads, a.k_max) > kNoAllocBytes) return SDI_ERR_TOO_LARGE;
    // the GPU the call runs on: the stream's (the current device for the null stream)
    int dev = 0;
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return SDI_ERR_HIP;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SDI_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SDI_ERR_HIP;
    void *base = nullptr;
    {
        // the array's address on that GPU, looked up once with that GPU current (host
        // code must not pass the array's name itself: on the host it is only a stand-in)
        std::lock_guard<std::mutex> lock(scratch_mu);
        if (!scratch_ptr[dev]) {
            int cur = 0;
            if (hipGetDevice(&cur) != hipSuccess) return SDI_ERR_HIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return SDI_ERR_HIP;
            void *p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev) (void)hipSetDevice(cur);
            if (e != hipSuccess || !p) return SDI_ERR_HIP;
            scratch_ptr[dev] = p;
        }
        base = scratch_ptr[dev];
    }
    a.ws = base;
    return launch_attend(a, stream) == hipSuccess ? SDI_OK : SDI_ERR_HIP;
}

}  // namespace sdi
