// softmax_kernels.hpp -- gfx950 (CDNA4) device code for the row-wise softmax
// of a binary16 matrix, the second memory-bound decode kernel of the
// "membound" page (section "Bonus kernel: online softmax").
//
//   y_ij = exp(x_ij - m_i) / d_i,  m_i = max_j x_ij,  d_i = sum_j exp(x_ij - m_i)
//
// The page's kernel finds m and d in one sweep with the online update
// (m' = max(m, x); d = d e^(m - m') + e^(x - m'), Milakov and Gimelshein) and
// normalises in a second pass that re-reads the row through L2.  Floor
// traffic is one read and one write of every element.
//
// Design here: a workgroup of W waves owns a row.  Each wave loads its units
// of the row (1 KiB per wave load, 8 binary16 per lane) into registers and
// sweeps them once with the online update, eight elements at a time (one
// rescale per eight); the lanes' (m, d) pairs merge with DPP butterflies,
// the waves' through LDS; the normalising pass then works from the same
// registers, so the row crosses HBM exactly once each way (rows up to
// W * UPW units; longer rows are read a second time).  All arithmetic is
// FP32; exp(t) is evaluated as 2^(t log2 e) with v_exp_f32, and the
// normalisation is folded into the exponent: y = 2^((x - m) log2 e - log2 d).
// Outputs are rounded to nearest even binary16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsoftmax {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr unsigned kNegInfPair = 0xFC00FC00u;   // two binary16 -inf

__device__ __forceinline__ float exp2_hw(float t) { return __builtin_amdgcn_exp2f(t); }
__device__ __forceinline__ float log2_hw(float t) { return __builtin_amdgcn_logf(t); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float a)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ float readlane(float v, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Combine two partial (max, normaliser) pairs.  An empty side has m = -inf
// and d = 0; using 0 in place of an infinite max keeps -inf - -inf out of
// the exponents (both factors are then 2^-inf = 0 or d is 0).  A NaN or +inf
// entry makes d NaN, which the normalising pass carries into every output.
__device__ __forceinline__ void merge(float& m, float& d, float m2, float d2)
{
    const float mn = fmaxf(m, m2);
    const float ms = mn == -__builtin_inff() ? 0.0f : mn;
    d = d * exp2_hw((m - ms) * kLog2e) + d2 * exp2_hw((m2 - ms) * kLog2e);
    m = mn;
}

template <int CTRL>
__device__ __forceinline__ void merge_dpp(float& m, float& d)
{
    merge(m, d, dpp_mov<CTRL>(m), dpp_mov<CTRL>(d));
}

// Merge the 64 lanes' pairs; the result is valid in every lane.
__device__ __forceinline__ void wave_merge(float& m, float& d)
{
    merge_dpp<0xB1>(m, d);    // lane ^ 1
    merge_dpp<0x4E>(m, d);    // lane ^ 2
    merge_dpp<0x141>(m, d);   // other quad of the 8-lane half row
    merge_dpp<0x140>(m, d);   // other half of the 16-lane row
    merge(m, d, swizzle_xor16(m), swizzle_xor16(d));   // lane ^ 16 within 32
    float m0 = readlane(m, 0), d0 = readlane(d, 0);
    merge(m0, d0, readlane(m, 32), readlane(d, 32));
    m = m0;
    d = d0;
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8])
{
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f16x2 h = __builtin_bit_cast(f16x2, w[k]);
        f[2 * k] = (float)h.x;
        f[2 * k + 1] = (float)h.y;
    }
}

// The online update over one 16-byte chunk: the chunk's own maximum, one
// rescale of d, eight exponentials against the new maximum.
__device__ __forceinline__ void sweep8(u32x4 v, float& m, float& d)
{
    float f[8];
    unpack8(v, f);
    float cm = fmaxf(fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])), fmaxf(fmaxf(f[4], f[5]), fmaxf(f[6], f[7])));
    const float mn = fmaxf(m, cm);
    const float ms = mn == -__builtin_inff() ? 0.0f : mn;
    float s = d * exp2_hw((m - ms) * kLog2e);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        s += exp2_hw((f[k] - ms) * kLog2e);
    d = s;
    m = mn;
}

// y for one chunk: 2^((x - m) log2 e - log2 d), rounded to binary16.
__device__ __forceinline__ u32x4 normalise8(u32x4 v, float m, float l2d)
{
    float f[8];
    unpack8(v, f);
    unsigned o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = exp2_hw(__builtin_fmaf(f[2 * k] - m, kLog2e, -l2d));
        const float b = exp2_hw(__builtin_fmaf(f[2 * k + 1] - m, kLog2e, -l2d));
        const f16x2 h = {(_Float16)a, (_Float16)b};
        o[k] = __builtin_bit_cast(unsigned, h);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// Preconditions (host): N % 8 == 0, N >= 8, x and y 16-byte aligned, M >= 1.
// One workgroup per row (grid-stride over rows); unit u of a row (64 chunks)
// belongs to wave u % W.  With PF, a workgroup whose row fits its registers
// loads its next row's units while it normalises and stores the current one
// (each register is reloaded right after its unit is stored), so the loads
// of the next row overlap the stores of this one.
template <int W, int UPW, bool PF>
__global__ void __launch_bounds__(W * 64)
softmax_f16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int N)
{
    __shared__ float red_m[W];
    __shared__ float red_d[W];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = N >> 3;
    const int P = (nchunks + 63) >> 6;
    constexpr int kSeg = W * UPW;
    const bool resident = P <= kSeg;
    u32x4 buf[UPW];
    auto load_unit = [&](const u32x4* src, int seg, int k) {
        const int c = (seg + k * W + wave) * 64 + lane;
        buf[k] = c < nchunks ? __builtin_nontemporal_load(src + c)
                             : u32x4{kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair};
    };
    bool preloaded = false;   // this row's units already in buf (PF)

    for (int row = blockIdx.x; row < M; row += gridDim.x) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)row * N);
        u32x4* dst = reinterpret_cast<u32x4*>(y + (int64_t)row * N);
        float m = -__builtin_inff(), d = 0.0f;
        for (int seg = 0; seg < P; seg += kSeg) {
            if (!preloaded) {
#pragma unroll
                for (int k = 0; k < UPW; ++k)
                    load_unit(src, seg, k);
            }
#pragma unroll
            for (int k = 0; k < UPW; ++k)
                sweep8(buf[k], m, d);
        }
        wave_merge(m, d);
        if (lane == 0) {
            red_m[wave] = m;
            red_d[wave] = d;
        }
        __syncthreads();
        m = red_m[0];
        d = red_d[0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            merge(m, d, red_m[w], red_d[w]);
        const float l2d = log2_hw(d);
        const int next = row + gridDim.x;
        const bool pf = PF && resident && next < M;
        const u32x4* nsrc = reinterpret_cast<const u32x4*>(x + (int64_t)(pf ? next : row) * N);
        for (int seg = 0; seg < P; seg += kSeg) {
            if (!resident) {
#pragma unroll
                for (int k = 0; k < UPW; ++k)
                    load_unit(src, seg, k);
            }
#pragma unroll
            for (int k = 0; k < UPW; ++k) {
                const int c = (seg + k * W + wave) * 64 + lane;
                if (c < nchunks)
                    __builtin_nontemporal_store(normalise8(buf[k], m, l2d), dst + c);
                if (pf)
                    load_unit(nsrc, 0, k);
            }
        }
        preloaded = pf;
        __syncthreads();   // the next row rewrites red_m / red_d
    }
}

// Any N and alignment: one wave per row, three passes with scalar loads
// (online max and normaliser, then outputs).  Waves walk rows 4 x gridDim.x
// apart (wave-uniform), so any grid covers them.
__global__ void __launch_bounds__(256)
softmax_f16_elementwise(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int N)
{
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < M; row += stride) {
        const _Float16* src = reinterpret_cast<const _Float16*>(x) + (int64_t)row * N;
        _Float16* dst = reinterpret_cast<_Float16*>(y) + (int64_t)row * N;
        float m = -__builtin_inff(), d = 0.0f;
#pragma unroll 8
        for (int64_t j = lane; j < N; j += 64)
            merge(m, d, (float)src[j], 1.0f);
        wave_merge(m, d);
        const float l2d = log2_hw(d);
#pragma unroll 8
        for (int64_t j = lane; j < N; j += 64)
            dst[j] = (_Float16)exp2_hw(__builtin_fmaf((float)src[j] - m, kLog2e, -l2d));
    }
}

}  // namespace gsoftmax
