// quant_kernels.hpp -- gfx950 (CDNA4) device code for the weight quantiser
// that produces the GEMV's INT8 and INT4 operands from FP32 weights.
//
// Formats ("membound", section "The kernel decode actually runs: dequant
// GEMV"): INT8 symmetric with one binary16 scale per row, INT4 symmetric
// with one binary16 scale per group of 128 columns, two's-complement nibbles
// two per byte with the even column in the low nibble.  Rule: scale =
// absmax / qmax (qmax 127 or 7) in binary32, rounded to binary16 (clamped to
// 65504); code = w / scale in binary32, rounded half to even, clipped to
// [-qmax, qmax]; a zero scale gives zero codes.  The squared error
// (q * scale - w)^2 is summed per row for the RMSE report.
//
// Both kernels read the FP32 weights once from HBM with 16-byte lane loads
// (4 weights per lane, 1 KiB per wave instruction) and write codes and
// scales once: a read-mostly stream (5 or 2.5 bytes moved per 4 input bytes).
//   * INT8 (a scale per row needs the whole row before the first code): one
//     workgroup per row; its waves load their share of the row into
//     registers, agree on the row maximum through LDS, then quantise from
//     registers.  Rows longer than the registers hold are read twice.
//   * INT4 (a scale per 128 columns): a group is 32 lanes' 16-byte chunks,
//     so one wave load holds two whole groups; the group maximum is a
//     32-lane butterfly and every unit is quantised as soon as it arrives.
//     Rows of up to 4 units: each wave streams whole rows with loads D
//     units ahead, like the GEMV.  Longer rows: a workgroup per row, its
//     waves taking every WAVES-th unit (no group spans two waves, so they
//     share nothing but the row's squared error, summed through LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gquant {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float as_f(unsigned w) { return __builtin_bit_cast(float, w); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float a)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v)
{
    // ds_swizzle bit mode, and_mask 0x1F, xor_mask 0x10: lane ^ 16 within 32
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Maximum over each 32-lane half of the wave; valid in every lane.
__device__ __forceinline__ float half_wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));    // lane ^ 1
    v = fmaxf(v, dpp_mov<0x4E>(v));    // lane ^ 2
    v = fmaxf(v, dpp_mov<0x141>(v));   // other quad of the 8-lane half row
    v = fmaxf(v, dpp_mov<0x140>(v));   // other half of the 16-lane row
    return fmaxf(v, swizzle_xor16(v));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = half_wave_max(v);
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return fmaxf(lo, hi);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    v += swizzle_xor16(v);
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return lo + hi;
}

__device__ __forceinline__ float absmax4(u32x4 v)
{
    return fmaxf(fmaxf(fabsf(as_f(v.x)), fabsf(as_f(v.y))), fmaxf(fabsf(as_f(v.z)), fabsf(as_f(v.w))));
}

// amax / qmax correctly rounded in binary32, for qmax 7 or 127 and amax >= 0,
// in three instructions instead of a full division: with r = RN(1/qmax),
// q = RN(amax r), the remainder e = amax - q qmax is exact in one FMA, and
// RN(q + e r) is the correctly rounded quotient for every finite amax >= 0
// (subnormals included) -- checked exhaustively for both constants against
// IEEE division.  An infinite amax gives e = NaN; then q (infinite) is the
// quotient; a NaN amax stays NaN.
template <int QMAX>
__device__ __forceinline__ float div_by_qmax(float amax)
{
    constexpr float kQ = (float)QMAX;
    constexpr float kR = 1.0f / kQ;
    const float q = amax * kR;
    const float e = __builtin_fmaf(-q, kQ, amax);
    const float y = __builtin_fmaf(e, kR, q);
    return y == y ? y : q;
}

// binary16 scale of a row or group: amax / qmax (correctly rounded binary32
// quotient), rounded to nearest even binary16 by v_cvt_f16_f32 (binary16
// subnormals kept), infinity clamped to 65504.  The maxima skip NaN weights;
// a row or group of NaN weights only has maximum 0 (v_max_f32 with 0 gives
// 0 for NaN), so its scale is 0.
template <int QMAX>
__device__ __forceinline__ uint16_t scale_bits(float amax)
{
    const float s = div_by_qmax<QMAX>(fmaxf(amax, 0.0f));
    uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)s);
    if (b == 0x7C00u)
        b = 0x7BFFu;
    return b;
}

__device__ __forceinline__ float half_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Code of one weight: the binary32 quotient w / sf rounded half to even
// (v_rndne_f32), clipped to [-QMAX, QMAX].  inv = 1 / sf from v_rcp_f32
// (once per row or group), or 0 when sf == 0.
//
// A correctly rounded division costs about ten VALU instructions, more than
// the memory stream leaves per weight, so the quotient is first taken as
// t = w * inv.  With inv within 2 ulp of 1 / sf (v_rcp_f32 is specified to
// 1 ulp, and measured within 0.82 ulp on every binary16 value), t differs from w / sf by at most 2^-22 + 2^-24 relative, and the
// correctly rounded quotient q from w / sf by 2^-24, so |t - q| is below
// 1.5 * 2^-22 * 128 < 2^-13 for |t| < 128.  Unless t lies within 2^-13 of a
// half-integer, every value that close rounds to the same integer as q
// does, so the fast result is exact; the rare weights near a half-integer
// take the correctly rounded division.  Values with |t| >= 128 clip to QMAX
// either way.  A NaN quotient (a NaN weight: the maxima skip NaN, so the
// scale is finite, possibly zero) fails the comparison below, so it too
// takes the rare path, which gives it code 0, as the oracle does; so does a
// zero scale there; an infinite weight takes it as well and clips.
template <int QMAX>
__device__ __forceinline__ float code_of(float w, float sf, float inv)
{
    float t = w * inv;
    const float frac = t - __builtin_floorf(t);
    if (__builtin_expect(!(__builtin_fabsf(frac - 0.5f) >= 0x1p-13f), 0)) {
        const float tq = sf != 0.0f ? w / sf : 0.0f;
        t = tq == tq ? tq : 0.0f;
    }
    const float r = __builtin_rintf(t);
    return fminf(fmaxf(r, -(float)QMAX), (float)QMAX);
}

__device__ __forceinline__ float inverse_of(float sf) { return sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f; }

// (q * sf - w)^2: q * sf is exact (at most 8 + 11 significant bits), so the
// FMA rounds only the difference.
__device__ __forceinline__ float sq_err(float q, float sf, float w)
{
    const float d = __builtin_fmaf(q, sf, -w);
    return d * d;
}

// ---------------------------------------------------------------- INT8
// Preconditions (host): N % 4 == 0, W 16-byte aligned, q 4-byte aligned,
// M >= 1, N >= 1.  One workgroup of WAVES waves per row (grid-stride over
// rows).  A row has P = ceil(N/256) units of 64 chunks; unit u belongs to
// wave u % WAVES.  With P <= WAVES * UPW the row stays in registers between
// the maximum and the codes; otherwise it is read a second time.
template <int WAVES, int UPW, bool SSE>
__global__ void __launch_bounds__(WAVES * 64)
quantize_q8_kernel(const float* __restrict__ W, int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                   float* __restrict__ row_sse, int M, int N)
{
    __shared__ float red_max[WAVES];
    __shared__ float red_sse[WAVES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = N >> 2;
    const int P = (nchunks + 63) >> 6;
    constexpr int kSeg = WAVES * UPW;       // units held per pass over the registers
    const bool resident = P <= kSeg;

    for (int row = blockIdx.x; row < M; row += gridDim.x) {
        const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)row * N);
        u32x4 buf[UPW];
        auto load_seg = [&](int seg) {
#pragma unroll
            for (int k = 0; k < UPW; ++k) {
                const int c = (seg + k * WAVES + wave) * 64 + lane;
                buf[k] = c < nchunks ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
            }
        };
        float amax = 0.0f;
        for (int seg = 0; seg < P; seg += kSeg) {
            load_seg(seg);
#pragma unroll
            for (int k = 0; k < UPW; ++k)
                amax = fmaxf(amax, absmax4(buf[k]));
        }
        amax = wave_max(amax);
        if (lane == 0)
            red_max[wave] = amax;
        __syncthreads();
        amax = red_max[0];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            amax = fmaxf(amax, red_max[w]);
        const uint16_t sb = scale_bits<127>(amax);
        const float sf = half_to_float(sb);
        const float inv = inverse_of(sf);
        if (threadIdx.x == 0)
            scale[row] = sb;

        float sse = 0.0f;
        uint32_t* dst = reinterpret_cast<uint32_t*>(q + (int64_t)row * N);
        for (int seg = 0; seg < P; seg += kSeg) {
            if (!resident)
                load_seg(seg);
#pragma unroll
            for (int k = 0; k < UPW; ++k) {
                const int c = (seg + k * WAVES + wave) * 64 + lane;
                if (c < nchunks) {
                    const float w0 = as_f(buf[k].x), w1 = as_f(buf[k].y), w2 = as_f(buf[k].z), w3 = as_f(buf[k].w);
                    const float c0 = code_of<127>(w0, sf, inv), c1 = code_of<127>(w1, sf, inv);
                    const float c2 = code_of<127>(w2, sf, inv), c3 = code_of<127>(w3, sf, inv);
                    if constexpr (SSE)
                        sse += sq_err(c0, sf, w0) + sq_err(c1, sf, w1) + sq_err(c2, sf, w2) + sq_err(c3, sf, w3);
                    dst[c] = ((uint32_t)(int)c0 & 0xFFu) | (((uint32_t)(int)c1 & 0xFFu) << 8) |
                             (((uint32_t)(int)c2 & 0xFFu) << 16) | ((uint32_t)(int)c3 << 24);
                }
            }
        }
        if constexpr (SSE) {
            sse = wave_sum(sse);
            if (lane == 0)
                red_sse[wave] = sse;
        }
        __syncthreads();   // also orders this row's reads of red_max before the next row's writes
        if (SSE && threadIdx.x == 0) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                t += red_sse[w];
            row_sse[row] = t;
        }
    }
}

// ---------------------------------------------------------------- INT4
// One INT4 unit of row `row`: lane `lane` holds chunk c (columns 4c..4c+3)
// of unit `unit` in v; lanes 0-31 hold the unit's first group, 32-63 its
// second.  Every lane takes part in the group maxima; only `live` lanes
// store codes (bytes 2c and 2c+1, the even column in the low nibble) and,
// lanes 0 and 32, the group scales.  Returns the lane's squared error (0
// unless SSE and live).
template <bool SSE>
__device__ __forceinline__ float q4_unit(const u32x4 v, int lane, int c, bool live, int row, int unit, int N,
                                         uint8_t* __restrict__ q, uint16_t* __restrict__ scale)
{
    const float amax = half_wave_max(absmax4(v));
    const uint16_t sb = scale_bits<7>(amax);
    const float sf = half_to_float(sb);
    const float inv = inverse_of(sf);
    const float w0 = as_f(v.x), w1 = as_f(v.y), w2 = as_f(v.z), w3 = as_f(v.w);
    const float c0 = code_of<7>(w0, sf, inv), c1 = code_of<7>(w1, sf, inv);
    const float c2 = code_of<7>(w2, sf, inv), c3 = code_of<7>(w3, sf, inv);
    float e = 0.0f;
    if (live) {
        if constexpr (SSE)
            e = sq_err(c0, sf, w0) + sq_err(c1, sf, w1) + sq_err(c2, sf, w2) + sq_err(c3, sf, w3);
        const uint32_t packed = ((uint32_t)(int)c0 & 0xFu) | (((uint32_t)(int)c1 & 0xFu) << 4) |
                                (((uint32_t)(int)c2 & 0xFu) << 8) | (((uint32_t)(int)c3 & 0xFu) << 12);
        reinterpret_cast<uint16_t*>(q + (int64_t)row * (N >> 1))[c] = (uint16_t)packed;
        if ((lane & 31) == 0)
            scale[(int64_t)row * (N >> 7) + unit * 2 + (lane >> 5)] = sb;
    }
    return e;
}

// Preconditions (host): N % 128 == 0, W 16-byte aligned, q 2-byte aligned,
// M >= 1.  Each wave owns rows wave_id, wave_id + nwaves, ... and walks
// their units (one 1-KiB wave load = two 128-column groups; a ragged last
// unit holds one group, in lanes 0..31) as one sequence, loads D units
// ahead.  The unit count is padded to a multiple of D; padded units re-read
// the wave's last row and store nothing.
template <int WAVES, int D, bool SSE>
__global__ void __launch_bounds__(WAVES * 64)
quantize_q4_kernel(const float* __restrict__ W, uint8_t* __restrict__ q, uint16_t* __restrict__ scale,
                   float* __restrict__ row_sse, int M, int N)
{
    const int lane = threadIdx.x & 63;
    const int nchunks = N >> 2;
    const int P = (nchunks + 63) >> 6;
    const int wave_id = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = gridDim.x * WAVES;
    const int my_rows = wave_id < M ? (M - 1 - wave_id) / nwaves + 1 : 0;
    const int units = my_rows * P;
    if (units == 0)
        return;
    const int units_pad = (units + D - 1) / D * D;
    const int last_row = wave_id + (my_rows - 1) * nwaves;

    u32x4 buf[D];
    int l_row = wave_id, l_pass = 0;
    auto issue = [&](int d) {
        const int row = l_row <= last_row ? l_row : last_row;
        const int c = l_pass * 64 + lane;
        const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)row * N);
        buf[d] = c < nchunks ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
        if (++l_pass == P) {
            l_pass = 0;
            l_row += nwaves;
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        issue(d);

    float sse = 0.0f;
    int c_row = wave_id, c_pass = 0;
    auto consume = [&](int d) {
        // padded units and lanes past the row store nothing
        const int c = c_pass * 64 + lane;
        const float e = q4_unit<SSE>(buf[d], lane, c, c_row < M && c < nchunks, c_row, c_pass, N, q, scale);
        if constexpr (SSE)
            sse += e;
        if (++c_pass == P) {
            if constexpr (SSE) {
                const float t = wave_sum(sse);
                if (lane == 0 && c_row < M)
                    row_sse[c_row] = t;
            }
            sse = 0.0f;
            c_pass = 0;
            c_row += nwaves;
        }
    };
    for (int k0 = D; k0 < units_pad; k0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            consume(d);
            issue(d);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        consume(d);
}

// Rows of many units: workgroup g quantises rows g, g + gridDim.x, ...;
// wave w takes the row's units w, w + WAVES, ... with loads D units ahead
// (within the row).  With SSE the waves' partial sums meet in LDS and one
// lane adds them in wave order, so the result does not depend on timing.
// Same preconditions as quantize_q4_kernel.
template <int WAVES, int D, bool SSE>
__global__ void __launch_bounds__(WAVES * 64)
quantize_q4_rows_kernel(const float* __restrict__ W, uint8_t* __restrict__ q, uint16_t* __restrict__ scale,
                        float* __restrict__ row_sse, int M, int N)
{
    __shared__ float red[WAVES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = N >> 2;
    const int P = (nchunks + 63) >> 6;
    const int k = P > wave ? (P - 1 - wave) / WAVES + 1 : 0;   // this wave's units in every row
    for (int row = blockIdx.x; row < M; row += gridDim.x) {
        const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)row * N);
        auto load = [&](int j) {   // this wave's j-th unit of the row
            const int c = (wave + j * WAVES) * 64 + lane;
            return c < nchunks ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
        };
        u32x4 buf[D];
#pragma unroll
        for (int d = 0; d < D; ++d)   // (a conditional load per d made the compiler wait for each in turn)
            buf[d] = d < k ? load(d) : u32x4{0u, 0u, 0u, 0u};
        float sse = 0.0f;
        for (int j0 = 0; j0 < k; j0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = j0 + d;
                if (j < k) {   // wave-uniform
                    const int u = wave + j * WAVES;
                    const int c = u * 64 + lane;
                    const float e = q4_unit<SSE>(buf[d], lane, c, c < nchunks, row, u, N, q, scale);
                    if constexpr (SSE)
                        sse += e;
                    if (j + D < k)
                        buf[d] = load(j + D);
                }
            }
        }
        if constexpr (SSE) {
            const float t = wave_sum(sse);
            if (lane == 0)
                red[wave] = t;
            __syncthreads();
            if (threadIdx.x == 0) {
                float r = 0.0f;
                for (int w = 0; w < WAVES; ++w)
                    r += red[w];
                row_sse[row] = r;
            }
            __syncthreads();   // red is reused by the next row
        }
    }
}

// ---------------------------------------------------------------- element-wise
// Any alignment and (INT8) any N: one wave per row, two passes with scalar
// loads (maximum, then codes).  INT4 still needs N % 128 == 0.  Waves walk
// rows 4 x gridDim.x apart, so any grid covers them.
template <int QMAX>
__global__ void __launch_bounds__(256)
quantize_elementwise_kernel(const float* __restrict__ W, uint8_t* __restrict__ q, uint16_t* __restrict__ scale,
                            float* __restrict__ row_sse, int M, int N)
{
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < M; row += stride) {   // wave-uniform
        const float* w = W + (int64_t)row * N;
        float sse = 0.0f;
        if constexpr (QMAX == 127) {
            float amax = 0.0f;
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                amax = fmaxf(amax, fabsf(w[j]));
            amax = wave_max(amax);
            const uint16_t sb = scale_bits<127>(amax);
            const float sf = half_to_float(sb);
            const float inv = inverse_of(sf);
            if (lane == 0)
                scale[row] = sb;
            int8_t* dst = reinterpret_cast<int8_t*>(q) + (int64_t)row * N;
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64) {
                const float c = code_of<127>(w[j], sf, inv);
                dst[j] = (int8_t)(int)c;
                sse += sq_err(c, sf, w[j]);
            }
        } else {
            // lane l handles byte pairs: columns 2b, 2b+1 for b = l, l+64, ...;
            // a group of 128 columns is 64 bytes, i.e. exactly one pass
            const int groups = N >> 7;
            uint8_t* dst = q + (int64_t)row * (N >> 1);
            for (int g = 0; g < groups; ++g) {
                const float a = w[g * 128 + 2 * lane], b = w[g * 128 + 2 * lane + 1];
                const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
                const uint16_t sb = scale_bits<7>(amax);
                const float sf = half_to_float(sb);
                const float inv = inverse_of(sf);
                if (lane == 0)
                    scale[(int64_t)row * groups + g] = sb;
                const float ca = code_of<7>(a, sf, inv), cb = code_of<7>(b, sf, inv);
                dst[g * 64 + lane] = (uint8_t)(((uint32_t)(int)ca & 0xFu) | (((uint32_t)(int)cb & 0xFu) << 4));
                sse += sq_err(ca, sf, a) + sq_err(cb, sf, b);
            }
        }
        const float t = wave_sum(sse);
        if (lane == 0 && row_sse != nullptr)
            row_sse[row] = t;
    }
}

}  // namespace gquant
