// Stochastic index selection on gfx950: uniform draws from the residual of a top-k row.
//
// The context-sparsity paper's German summary (sections 2 and 3A) evaluates
// vAttention's stochastic selection next to exact top-k; the estimator itself is not
// on the pages, and the library takes the plain Monte Carlo reading.  A row keeps its
// top-k set S; s' further tokens are drawn uniformly, with replacement, from the
// residual R = [0, N_b) \ S of M tokens, and each drawn token enters the softmax sums
// with weight M / s' (the attend launch's two-list mode).  The random numbers are
// inputs: draw x (32 bits) picks residual rank r = floor(x M / 2^32).
//
// Rank to token: with S ascending (s_0 < s_1 < ...), exactly s_i - i residual tokens
// lie below s_i, and s_i - i never decreases; the r-th residual token is r + c with
// c = #{i : s_i - i <= r}, found by bisection.  One workgroup per (b, h): the kept
// row is staged in LDS (rows of up to 15360 entries, 60 KB; longer ones are
// searched in place), counted, and each thread maps its draws.  The work is a few KB per row:
// latency, not bandwidth, bounds it.
#include "sdi_device.hpp"
#include "sdi_launch.hpp"

namespace sdi {

constexpr int kSampleThreads = 256;
constexpr int kSampleLdsMax = 15360;     // staged rows stay within 64 KB of LDS

// grid (num_q_heads, batch); dynamic LDS min(k_max, kSampleLdsMax) ints.
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ k_per_seq, int k_max,
    const int32_t *__restrict__ seq_lens, int num_q_heads, const uint32_t *__restrict__ draws,
    const int32_t *__restrict__ s_per_seq, int s_max, int32_t *__restrict__ sample_out,
    float *__restrict__ weight_out)
{
    extern __shared__ int32_t row_lds[];
    __shared__ int kept_count;
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const int n = max(seq_lens[b], 0);
    const int kk = max(min(k_per_seq[b], k_max), 0);
    const int32_t *grow = idx + bh * k_max;
    const bool staged = k_max <= kSampleLdsMax;

    if (threadIdx.x == 0) kept_count = 0;
    __syncthreads();
    int cnt = 0;
    for (int i = threadIdx.x; i < kk; i += kSampleThreads) {
        const int j = grow[i];
        cnt += (j >= 0 && j < n);
        if (staged) row_lds[i] = j;
    }
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&kept_count, cnt);
    __syncthreads();

    // The kept tokens are entries [0, kp) of the row, ascending (the top-k row format).
    const int kp = kept_count;
    const int M = n - kp;
    int s = min(s_per_seq[b], s_max);
    if (s < 0 || M <= 0) s = 0;
    if (threadIdx.x == 0) weight_out[bh] = s > 0 ? (float)M / (float)s : 0.f;
    const int32_t *row = staged ? row_lds : grow;
    for (int t = threadIdx.x; t < s_max; t += kSampleThreads) {
        int tok = -1;
        if (t < s) {
            const int r = (int)(((uint64_t)draws[bh * s_max + t] * (uint64_t)M) >> 32);
            int lo = 0, hi = kp;                       // count entries with s_i - i <= r
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (row[mid] - mid <= r) lo = mid + 1;
                else hi = mid;
            }
            tok = r + lo;
        }
        sample_out[bh * s_max + t] = tok;
    }
}

hipError_t launch_sample(const SampleArgs &a, hipStream_t stream)
{
    const size_t lds = (size_t)std::min(a.k_max, kSampleLdsMax) * sizeof(int32_t);
    hipLaunchKernelGGL(sample_kernel, dim3(a.num_q_heads, a.batch), dim3(kSampleThreads), lds, stream, a.idx,
                       a.k_per_seq, a.k_max, a.seq_lens, a.num_q_heads, a.draws, a.s_per_seq, a.s_max,
                       a.sample_out, a.weight_out);
    return hipGetLastError();
}

}  // namespace sdi
