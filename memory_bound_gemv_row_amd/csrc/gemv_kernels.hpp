// gemv_kernels.hpp -- gfx950 (CDNA4) device code for row-major GEMV.
//
//   y_i = sum_j A_ij x_j,  A row-major: element (i, j) at offset i*N + j
//   ("Making GEMV Fast", sections "Algorithm" and "Row-major indexing
//   refresher").
//
// Design (wave64, one pass of HBM over A):
//   * A wave owns R rows at a time ("Making GEMV Fast", section "What access
//     pattern do we actually want?": give a row to a warp, not a thread).
//     Lane l reads the 16-byte chunks l, l+64, l+128, ... of each row, so one
//     wave-wide load instruction moves 1 KiB of contiguous bytes: the
//     coalesced mapping "column = lane + width * pass" at 16-byte
//     granularity ("membound", stage 3: 128-bit loads).
//   * U chunks per lane and row are issued before any is consumed, so each
//     wave keeps U*R KiB of A in flight.
//   * x is staged once per workgroup in LDS ("membound", stage 2 stages x in
//     shared memory), or, when it does not fit, read through the caches.
//   * Accumulation is FP32 in registers.  FP16 operands enter through
//     v_dot2_f32_f16; INT8/INT4 codes are unpacked in registers to exact
//     binary16 integers (exponent-bias trick, below) and enter the same way;
//     the INT8 row scale multiplies the finished row sum, the INT4 group scale
//     multiplies each 32-column partial (the reference weight is exactly
//     q*s: "membound", section "The kernel decode actually runs: dequant
//     GEMV").
//   * The 64 lane partials are combined with DPP and ds_swizzle steps; no
//     LDS round trip and no atomics ("Making GEMV Fast", section "How does
//     warpReduceSum work?", and the llama.cpp walkthrough's butterfly, both
//     on 32-wide warps; here the butterfly spans 64 lanes).  Lane 0 stores.
//
// No MFMA: at batch 1 each weight is used once, so the work is a stream of
// about one FMA per weight, bounded by HBM bandwidth, not a contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum Format : int { kF32 = 0, kF16 = 1, kQ8 = 2, kQ4 = 3 };

// Per-format geometry of one 16-byte chunk of A.
//   kElems : matrix elements per chunk
//   kXGran : 16-byte granules of x that those elements need
template <int F> struct Traits;
template <> struct Traits<kF32> { static constexpr int kElems = 4;  static constexpr int kXGran = 1; };
template <> struct Traits<kF16> { static constexpr int kElems = 8;  static constexpr int kXGran = 1; };
template <> struct Traits<kQ8>  { static constexpr int kElems = 16; static constexpr int kXGran = 2; };
template <> struct Traits<kQ4>  { static constexpr int kElems = 32; static constexpr int kXGran = 4; };

__device__ __forceinline__ f16x2 as_h2(unsigned w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ float as_f(unsigned w) { return __builtin_bit_cast(float, w); }

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// ---------------------------------------------------------------- reduction
// Sum of v over the 64 lanes of the wave; valid in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float a)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_mov<0x141>(v);  // row_half_mirror: other quad of the 8-lane half row
    v += dpp_mov<0x140>(v);  // row_mirror: other half of the 16-lane row
    // ds_swizzle bit mode, and_mask 0x1F, xor_mask 0x10: lane ^ 16 within 32
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return lo + hi;
}

// ---------------------------------------------------------------- chunk products
// Each returns acc plus the dot product of one 16-byte chunk of A with the
// matching x elements.  Products are exact in FP32 for every format (at most
// 24 significant bits); only the additions round.

// FP32: 4 columns.
__device__ __forceinline__ float chunk_f32(u32x4 a, u32x4 xv, float acc)
{
    acc = __builtin_fmaf(as_f(a.x), as_f(xv.x), acc);
    acc = __builtin_fmaf(as_f(a.y), as_f(xv.y), acc);
    acc = __builtin_fmaf(as_f(a.z), as_f(xv.z), acc);
    acc = __builtin_fmaf(as_f(a.w), as_f(xv.w), acc);
    return acc;
}

// FP16: 8 columns, pairs (2k, 2k+1) through v_dot2_f32_f16.
__device__ __forceinline__ float chunk_f16(u32x4 a, u32x4 xv, float acc)
{
    acc = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(xv.w), acc, false);
    return acc;
}

// INT8 -> exact binary16 integer.  Flipping the sign bit turns the
// two's-complement code q into the unsigned byte q + 128; placed under the
// binary16 exponent of 1024 (bits 0x64xx) that byte becomes the value
// 1024 + q + 128, exactly, since binary16 spacing in [1024, 2048) is 1.
// Subtracting 1152 leaves q.  Two columns per 32-bit register.
__device__ __forceinline__ float q8_word(unsigned w, unsigned x01, unsigned x23, float acc)
{
    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    w ^= 0x80808080u;
    const unsigned b01 = (w & 0x000000FFu) | ((w << 8) & 0x00FF0000u) | 0x64006400u;
    const unsigned b23 = ((w >> 16) & 0x000000FFu) | ((w >> 8) & 0x00FF0000u) | 0x64006400u;
    acc = __builtin_amdgcn_fdot2(as_h2(b01) + bias, as_h2(x01), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(b23) + bias, as_h2(x23), acc, false);
    return acc;
}

// INT8: 16 columns; x0 holds columns 0..7, x1 columns 8..15 (binary16).
__device__ __forceinline__ float chunk_q8(u32x4 a, u32x4 x0, u32x4 x1, float acc)
{
    acc = q8_word(a.x, x0.x, x0.y, acc);
    acc = q8_word(a.y, x0.z, x0.w, acc);
    acc = q8_word(a.z, x1.x, x1.y, acc);
    acc = q8_word(a.w, x1.z, x1.w, acc);
    return acc;
}

// INT4 -> exact binary16 integers.  One 32-bit word holds columns c..c+7,
// column c+k in bits [4k, 4k+4).  XOR with 0x8 per nibble turns a
// two's-complement code q into q + 8 in 0..15.  Masking with 0x000F000F
// keeps columns c and c+4 in the low mantissa bits of the two binary16
// halves; under exponent bits 0x6400 they read 1024 + (q + 8), and
// subtracting 1032 leaves q.  Mask 0x00F000F0 keeps columns c+1 and c+5 four
// bits higher: 1024 + 16(q + 8), minus 1152, is 16q (exact), and the factor
// 16 is removed once per chunk.  Shifting the word right by 8 gives columns
// c+2, c+6 and c+3, c+7 the same way.  x is therefore staged with each
// 8-column block reordered as (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ void q4_word(unsigned w, u32x4 xp, float& acc_1, float& acc_16)
{
    const f16x2 b1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 b16 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    w ^= 0x88888888u;
    const unsigned w8 = w >> 8;
    acc_1 = __builtin_amdgcn_fdot2(as_h2((w & 0x000F000Fu) | 0x64006400u) + b1, as_h2(xp.x), acc_1, false);
    acc_16 = __builtin_amdgcn_fdot2(as_h2((w & 0x00F000F0u) | 0x64006400u) + b16, as_h2(xp.y), acc_16, false);
    acc_1 = __builtin_amdgcn_fdot2(as_h2((w8 & 0x000F000Fu) | 0x64006400u) + b1, as_h2(xp.z), acc_1, false);
    acc_16 = __builtin_amdgcn_fdot2(as_h2((w8 & 0x00F000F0u) | 0x64006400u) + b16, as_h2(xp.w), acc_16, false);
}

// INT4: 32 columns (all inside one 128-column group) and their group scale.
__device__ __forceinline__ float chunk_q4(u32x4 a, const u32x4 (&xp)[4], float s, float acc)
{
    float acc_1 = 0.0f, acc_16 = 0.0f;
    q4_word(a.x, xp[0], acc_1, acc_16);
    q4_word(a.y, xp[1], acc_1, acc_16);
    q4_word(a.z, xp[2], acc_1, acc_16);
    q4_word(a.w, xp[3], acc_1, acc_16);
    return __builtin_fmaf(s, __builtin_fmaf(acc_16, 0.0625f, acc_1), acc);
}

// Reorder one 8-column block of binary16 x from (x0..x7) to
// (x0,x4), (x1,x5), (x2,x6), (x3,x7), the pairing q4_word expects.
__device__ __forceinline__ u32x4 q4_pair_x(u32x4 v)
{
    u32x4 r;
    r.x = (v.x & 0xFFFFu) | (v.z << 16);
    r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    r.z = (v.y & 0xFFFFu) | (v.w << 16);
    r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return r;
}

// ---------------------------------------------------------------- bandwidth kernel
// Preconditions (checked by the host): N is a multiple of Traits<F>::kElems,
// A and x are 16-byte aligned, M >= 1.  For XLDS the launch provides
// N * sizeof(x element) bytes of dynamic LDS.
template <int F, int WAVES, int R, int U, bool XLDS, bool NT>
__global__ void __launch_bounds__(WAVES * 64)
gemv_rows(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
          const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    using T = Traits<F>;
    extern __shared__ u32x4 lds_x[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nchunks = N / T::kElems;
    const int64_t row_bytes = (int64_t)nchunks * 16;
    const u32x4* xg = reinterpret_cast<const u32x4*>(x);

    if constexpr (XLDS) {
        const int nxg = nchunks * T::kXGran;
        for (int g = threadIdx.x; g < nxg; g += WAVES * 64) {
            u32x4 v = xg[g];
            if constexpr (F == kQ4)
                v = q4_pair_x(v);
            lds_x[g] = v;
        }
        __syncthreads();
    }

    auto xgran = [&](int g) -> u32x4 {
        if constexpr (XLDS) {
            return lds_x[g];
        } else {
            u32x4 v = xg[g];
            if constexpr (F == kQ4)
                v = q4_pair_x(v);
            return v;
        }
    };

    const int ngroups = (M + R - 1) / R;
    const int groups_per_row_scale = N / 128;   // INT4 scales per row
    for (int grp = blockIdx.x * WAVES + wave; grp < ngroups; grp += gridDim.x * WAVES) {
        const int row0 = grp * R;
        const u32x4* arow[R];
        int rclamp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // rows past M re-read row M-1 (in bounds); their sums are dropped
            rclamp[r] = min(row0 + r, M - 1);
            arow[r] = reinterpret_cast<const u32x4*>(A + (int64_t)rclamp[r] * row_bytes);
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0.0f;

        for (int c0 = 0; c0 < nchunks; c0 += 64 * U) {
            u32x4 a[U][R];
            float s[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * 64 + lane;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    a[u][r] = (c < nchunks) ? load16<NT>(arow[r] + c) : u32x4{0u, 0u, 0u, 0u};
                    if constexpr (F == kQ4)
                        s[u][r] = (c < nchunks)
                            ? half_bits_to_float(scale[(int64_t)rclamp[r] * groups_per_row_scale + (c >> 2)])
                            : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nchunks) {
                    if constexpr (F == kF32) {
                        const u32x4 xv = xgran(c);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r] = chunk_f32(a[u][r], xv, acc[r]);
                    } else if constexpr (F == kF16) {
                        const u32x4 xv = xgran(c);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r] = chunk_f16(a[u][r], xv, acc[r]);
                    } else if constexpr (F == kQ8) {
                        const u32x4 x0 = xgran(2 * c), x1 = xgran(2 * c + 1);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r] = chunk_q8(a[u][r], x0, x1, acc[r]);
                    } else {
                        const u32x4 xp[4] = {xgran(4 * c), xgran(4 * c + 1), xgran(4 * c + 2), xgran(4 * c + 3)};
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r] = chunk_q4(a[u][r], xp, s[u][r], acc[r]);
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r) {
            float t = wave_sum(acc[r]);
            if (lane == 0 && row0 + r < M) {
                if constexpr (F == kQ8)
                    t *= half_bits_to_float(scale[row0 + r]);
                y[row0 + r] = t;
            }
        }
    }
}

// ---------------------------------------------------------------- element-wise kernel
// Any N >= 0 and any alignment: one wave per row, lane l takes columns
// l, l+64, ... with scalar loads (INT4: bytes l, l+64, ..., two columns
// each).  Four waves per workgroup.
template <int F>
__global__ void __launch_bounds__(256)
gemv_elementwise(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
                 const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M)
        return;   // whole wave leaves together
    float acc = 0.0f;
    if constexpr (F == kF32) {
        const float* a = reinterpret_cast<const float*>(A) + (int64_t)row * N;
        const float* xf = reinterpret_cast<const float*>(x);
        for (int j = lane; j < N; j += 64)
            acc = __builtin_fmaf(a[j], xf[j], acc);
    } else if constexpr (F == kF16) {
        const uint16_t* a = reinterpret_cast<const uint16_t*>(A) + (int64_t)row * N;
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
        for (int j = lane; j < N; j += 64)
            acc = __builtin_fmaf(half_bits_to_float(a[j]), half_bits_to_float(xh[j]), acc);
    } else if constexpr (F == kQ8) {
        const int8_t* a = reinterpret_cast<const int8_t*>(A) + (int64_t)row * N;
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
        for (int j = lane; j < N; j += 64)
            acc = __builtin_fmaf((float)a[j], half_bits_to_float(xh[j]), acc);
    } else {
        const int half_n = N / 2;
        const uint8_t* a = A + (int64_t)row * half_n;
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
        const uint16_t* srow = scale + (int64_t)row * (N / 128);
        for (int b = lane; b < half_n; b += 64) {
            const unsigned byte = a[b];
            const int q0 = (int)(byte & 0xFu) - (int)((byte & 0x8u) << 1);
            const int q1 = (int)(byte >> 4) - (int)((byte & 0x80u) >> 3);
            const float s = half_bits_to_float(srow[(2 * b) >> 7]);
            acc = __builtin_fmaf((float)q0 * s, half_bits_to_float(xh[2 * b]), acc);
            acc = __builtin_fmaf((float)q1 * s, half_bits_to_float(xh[2 * b + 1]), acc);
        }
    }
    float t = wave_sum(acc);
    if (lane == 0) {
        // N == 0 is the empty sum: y = 0 whatever the scale (which is not read)
        if constexpr (F == kQ8)
            if (N > 0)
                t *= half_bits_to_float(scale[row]);
        y[row] = t;
    }
}

// ---------------------------------------------------------------- probes
// Pure-read stream: each workgroup reads U*WG consecutive 16-byte granules
// per step, then strides over the grid.
template <int U, bool NT>
__global__ void __launch_bounds__(256)
probe_read_kernel(const u32x4* __restrict__ buf, int64_t n16, uint32_t* __restrict__ sink, uint32_t guard)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = (i < n16) ? load16<NT>(buf + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u];
    }
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == guard)
        sink[0] = f;
}

template <int U, bool NT>
__global__ void __launch_bounds__(256)
probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n16)
                v[u] = load16<NT>(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n16)
                dst[i] = v[u];
        }
    }
}

}  // namespace gemv
