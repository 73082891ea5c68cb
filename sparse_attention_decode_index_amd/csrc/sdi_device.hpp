// Device helpers shared by the gfx950 kernels: bf16 unpacking, 16-lane DPP
// reductions, the order-preserving score key, a workgroup scan and the MFMA
// operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdi {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kRowBytes = kHeadDim * 2;        // one bf16 row
constexpr int kHistBits = 12;                  // first radix digit of a key (counted by the score pass)
constexpr int kHistBins = 1 << kHistBits;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Unpack 8 bf16 (one 16-byte load) to fp32.
__device__ __forceinline__ void unpack8(const u32x4 &w, float *f)
{
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Monotone map of an fp32 score to uint32: a larger score gives a larger key.
// -0 is folded into +0 so that equal scores always give equal keys.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each half row
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each row

// Sum / max over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row_shr 1/2/4/8 inside
// each 16-lane row, then row_bcast 15 (into rows 1 and 3) and row_bcast 31 (into rows
// 2 and 3).  Lanes whose DPP source does not exist receive 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64).
// `scratch` needs NT/64 words of LDS.  Returns this thread's exclusive prefix and
// sets `total`.  Contains two workgroup barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        uint32_t t = scratch[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight
// (a full __syncthreads also waits for every vector memory operation).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace sdi
