// gemv_kernels.hpp -- gfx950 (CDNA4) device code for row-major GEMV.
//
//   y_i = sum_j A_ij x_j,  A row-major: element (i, j) at offset i*N + j
//   ("Making GEMV Fast", sections "Algorithm" and "Row-major indexing
//   refresher").
//
// Design (wave64, one pass of HBM over A):
//   * A wave owns whole rows ("Making GEMV Fast", section "What access
//     pattern do we actually want?": give a row to a warp, not a thread).
//     Lane l reads the 16-byte chunks l, l+64, l+128, ... of each row, so one
//     wave-wide load instruction moves 1 KiB of contiguous bytes: the
//     coalesced mapping "column = lane + width * pass" at 16-byte
//     granularity ("membound", stage 3: 128-bit loads).  Rows shorter than
//     half a wave load share wave loads (gemv_packed); few long rows, and
//     INT8/INT4/FP16-with-FP32-x rows in slabs of 4 or 8, spread one row's
//     passes over the waves of a workgroup (gemv_split, gemv_slab).
//   * D such 1-KiB units are issued before any is consumed, so each wave
//     keeps D KiB of A in flight.
//   * x reaches the lanes one of three ways, by shape: staged once per
//     workgroup in LDS ("membound", stage 2 stages x in shared memory), read
//     through the caches with each unit, or loaded once per wave into
//     registers: for rows of one to three wave loads, packed short rows, and
//     in row slabs each wave's slice of x for the passes it owns.
//   * Accumulation is FP32 in registers.  FP16 operands enter through
//     v_dot2_f32_f16; INT8/INT4 codes are unpacked in registers to exact
//     binary16 integers (INT8 by a byte-select conversion, INT4 through an
//     exponent bias, below) and enter the same way; the INT8 row scale multiplies
//     the finished row sum, the INT4 group scale multiplies each 32-column
//     partial (the reference weight is exactly q*s: "membound", section "The
//     kernel decode actually runs: dequant GEMV").  FP16 weights with FP32 x
//     use v_fma_mix_f32; the FP16-accumulation entry point keeps binary16
//     running sums (v_pk_fma_f16).
//   * The 64 lane partials are combined with DPP and ds_swizzle steps; no
//     LDS round trip and no atomics ("Making GEMV Fast", section "How does
//     warpReduceSum work?", and the llama.cpp walkthrough's butterfly, both
//     on 32-wide warps; here the butterfly spans 64 lanes).  Lane 0 stores.
//     Row slabs reduce four or eight rows' partials at once with lane
//     permutes, and a row whose passes span waves meets in LDS.
//
// No MFMA: at batch 1 each weight is used once, so the work is a stream of
// about one FMA per weight, bounded by HBM bandwidth, not a contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// kF16X32: binary16 A with an FP32 x (the hidden state kept in FP32).
// kF16H: binary16 A and x with binary16 running sums (lossy; see chunk_f16h).
enum Format : int { kF32 = 0, kF16 = 1, kQ8 = 2, kQ4 = 3, kF16X32 = 4, kF16H = 5 };

// Per-format geometry of one 16-byte chunk of A.
//   kElems : matrix elements per chunk
//   kXGran : 16-byte granules of x that those elements need
template <int F> struct Traits;
template <> struct Traits<kF32> { static constexpr int kElems = 4;  static constexpr int kXGran = 1; };
template <> struct Traits<kF16> { static constexpr int kElems = 8;  static constexpr int kXGran = 1; };
template <> struct Traits<kF16X32> { static constexpr int kElems = 8; static constexpr int kXGran = 2; };
template <> struct Traits<kF16H> { static constexpr int kElems = 8;  static constexpr int kXGran = 1; };
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
// matching x elements.  Only the additions round: FP32 and FP16-with-FP32-x
// products are formed inside an FMA, which rounds once after the add, and
// the other formats' products have at most 24 significant bits.

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

// FP16 with FP16 accumulation: 8 columns into one pair of binary16 running
// sums (even columns in .x, odd in .y), one v_pk_fma_f16 per column pair,
// so each term costs one binary16 rounding.  The caller widens the pair to
// FP32 at the row end; the cross-lane reduction and y are FP32.  Lossy: a
// lane's sums carry N/128 terms each at binary16 precision and overflow
// past 65504.
__device__ __forceinline__ f16x2 chunk_f16h(u32x4 a, u32x4 xv, f16x2 acc)
{
    acc = __builtin_elementwise_fma(as_h2(a.x), as_h2(xv.x), acc);
    acc = __builtin_elementwise_fma(as_h2(a.y), as_h2(xv.y), acc);
    acc = __builtin_elementwise_fma(as_h2(a.z), as_h2(xv.z), acc);
    acc = __builtin_elementwise_fma(as_h2(a.w), as_h2(xv.w), acc);
    return acc;
}

// FP16 A with FP32 x: 8 columns; x0 holds columns 0..3, x1 columns 4..7.
// Each binary16 weight is widened exactly and meets its FP32 x in one FMA
// (v_fma_mix_f32 selects the low or high half of the A register), so every
// product is exact and only the additions round, as in the FP32 path.
__device__ __forceinline__ float chunk_f16x32(u32x4 a, u32x4 x0, u32x4 x1, float acc)
{
    const unsigned ws[4] = {a.x, a.y, a.z, a.w};
    const unsigned xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f16x2 h = as_h2(ws[k]);
        acc = __builtin_fmaf((float)h.x, as_f(xs[2 * k]), acc);
        acc = __builtin_fmaf((float)h.y, as_f(xs[2 * k + 1]), acc);
    }
    return acc;
}

// INT4 -> exact binary16 integers.  One 32-bit word holds columns c..c+7,
// column c+k in bits [4k, 4k+4).  XOR with 0x8 per nibble turns a
// two's-complement code q into q + 8 in 0..15.  Masking with 0x000F000F
// keeps columns c and c+4 in the low mantissa bits of the two binary16
// halves; under exponent bits 0x6400 (2^10, unit spacing) they read
// 1024 + (q + 8), and subtracting 1032 leaves q.  Mask 0x00F000F0 keeps
// columns c+1 and c+5 four bits higher; under exponent bits 0x5400 (2^6,
// spacing 1/16) they read 64 + (q + 8), and subtracting 72 leaves q.  Each
// mask-and-XOR is one v_bitop3_b32 and each subtraction one v_pk_add_f16,
// exact.  Shifting the word right by 8 gives columns c+2, c+6 and c+3, c+7
// the same way.  x is therefore staged with each 8-column block reordered
// as (x0,x4), (x1,x5), (x2,x6), (x3,x7).  All four pairs enter one FP32 sum.
__device__ __forceinline__ float q4_word(unsigned w, u32x4 xp, float acc)
{
    const f16x2 b_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 b_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    // (w ^ 0x88888888) & mask | exponent bits, written as one AND and one
    // XOR: the XOR constant flips the nibble's sign bit (bit 3 or bit 7 of
    // each half) and sets the exponent bits, which the mask has cleared
    const unsigned w8 = w >> 8;
    acc = __builtin_amdgcn_fdot2(as_h2((w & 0x000F000Fu) ^ 0x64086408u) + b_lo, as_h2(xp.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w & 0x00F000F0u) ^ 0x54805480u) + b_hi, as_h2(xp.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w8 & 0x000F000Fu) ^ 0x64086408u) + b_lo, as_h2(xp.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w8 & 0x00F000F0u) ^ 0x54805480u) + b_hi, as_h2(xp.w), acc, false);
    return acc;
}

// INT4: 32 columns (all inside one 128-column group) and their group scale.
__device__ __forceinline__ float chunk_q4(u32x4 a, const u32x4 (&xp)[4], float s, float acc)
{
    float part = 0.0f;
    part = q4_word(a.x, xp[0], part);
    part = q4_word(a.y, xp[1], part);
    part = q4_word(a.z, xp[2], part);
    part = q4_word(a.w, xp[3], part);
    return __builtin_fmaf(s, part, acc);
}

// INT8 -> exact binary16 pairs.  v_cvt_f16_i16 with an SDWA source select
// converts one sign-extended byte of the word to binary16; the first
// conversion writes the low half (clearing the high one), the second writes
// the high half and keeps the low.  Every code is an integer of magnitude at
// most 128, so each binary16 value is the code itself, and v_dot2_f32_f16
// then forms each product q*x exactly: the row sum carries no offset to
// cancel, whatever x holds (the reference weight is exactly q*s: "membound",
// section "The kernel decode actually runs: dequant GEMV").
__device__ __forceinline__ unsigned q8_pair_lo(unsigned w)
{
    unsigned r;
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1"
        : "=&v"(r)
        : "v"(w));
    return r;
}

__device__ __forceinline__ unsigned q8_pair_hi(unsigned w)
{
    unsigned r;
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "=&v"(r)
        : "v"(w));
    return r;
}

// INT8 chunk: acc + sum q x over 16 columns; bytes (2k, 2k+1) of the chunk
// meet x's natural pairs.
__device__ __forceinline__ float q8_chunk(u32x4 a, u32x4 x0, u32x4 x1, float acc)
{
    const unsigned ws[4] = {a.x, a.y, a.z, a.w};
    const unsigned xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc = __builtin_amdgcn_fdot2(as_h2(q8_pair_lo(ws[k])), as_h2(xs[2 * k]), acc, false);
        acc = __builtin_amdgcn_fdot2(as_h2(q8_pair_hi(ws[k])), as_h2(xs[2 * k + 1]), acc, false);
    }
    return acc;
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

// Where granule k (of kXGran) of chunk c sits in staged x.  The LDS serves
// a 16-byte read to 16 lanes per clock from 64 four-byte banks, so a wave's
// read of one granule per lane is conflict-free only where the lanes' 16
// bytes are consecutive.  FP16-with-FP32-x stores each of its two granules
// as its own plane of nchunks_pad granules.  INT4 (four granules, 64 bytes
// per chunk: x's natural order put 4 of each 16 lanes on the same banks)
// keeps the chunks of each pass together and splits them by granule: the
// four reads of a unit are 1 KiB apart, an offset the LDS instruction holds,
// so planes cost no address arithmetic (14336 x 4096: 1.4 M bank-conflict
// cycles per launch to 0.2 M, all of them the staging writes', median 7.68
// -> 7.19 us; 4096 x 14336 8.06 -> 7.94).  INT8 keeps x's natural order (two granules per chunk, 2-way
// conflicts): neither kind of plane measured faster for it.
template <int F>
__device__ __forceinline__ int staged_index(int c, int k, int nchunks_pad)
{
    constexpr int G = Traits<F>::kXGran;
    if constexpr (F == kF16X32)
        return k * nchunks_pad + c;
    else if constexpr (F == kQ4)
        return ((c >> 6) * G + k) * 64 + (c & 63);
    else
        return c * G + k;
}

// Copy the nxg 16-byte granules of x into LDS in the staged order
// (staged_index; INT4: each granule reordered for q4_word).  Each thread issues up to 8
// loads before the first wait, so staging costs about one cache round trip
// per 8 granules.
template <int F, int NT>
__device__ __forceinline__ void stage_x(const u32x4* __restrict__ xg, u32x4* lds, int nxg, int nxg_pad)
{
    constexpr int G = Traits<F>::kXGran;
    const int nchunks_pad = nxg_pad / G;
    for (int g0 = threadIdx.x; g0 < nxg_pad; g0 += 8 * NT) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int g = g0 + k * NT;
            v[k] = xg[g < nxg ? g : 0];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int g = g0 + k * NT;
            if (g >= nxg_pad)
                continue;
            const int dst = staged_index<F>(g / G, g % G, nchunks_pad);
            if (g < nxg)
                lds[dst] = (F == kQ4) ? q4_pair_x(v[k]) : v[k];
            else
                lds[dst] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Split staging (see default_stage_order): rounds of split_round<F>()
// granules per thread, granule g = g0 + k * NT for k < that.  Neither the loads
// nor the LDS writes branch per granule: a load or store under a condition
// compiles to a branch, after which the compiler no longer knows which loads
// are in flight and waits for all of them, the A loads included, before the
// write.  So every load is issued (granule 0 stands in past x's end and is
// zeroed), and every write happens: granules past the zero-padded end go to
// one spare granule per lane after the staged x (kSplitSpareBytes more LDS).
// Granules per thread in a round: INT8 and INT4 split rows of a few units
// (one to three granules per thread), FP16 with FP32 x rows up to 32 units
// (up to eight); a larger round only adds loads of granule 0 and spare writes.
template <int F>
__host__ __device__ constexpr int split_round()
{
#ifdef GEMV_SPLIT_ROUND
    return GEMV_SPLIT_ROUND;
#else
    return F == kF16X32 ? 8 : 2;
#endif
}
constexpr int kSplitSpareBytes = 64 * 16;

template <int F, int NT>
__device__ __forceinline__ void split_round_load(const u32x4* __restrict__ xg, int g0, int nxg,
                                                 u32x4 (&v)[split_round<F>()])
{
#pragma unroll
    for (int k = 0; k < split_round<F>(); ++k) {
        const int g = g0 + k * NT;
        v[k] = xg[g < nxg ? g : 0];
    }
}

template <int F, int NT>
__device__ __forceinline__ void split_round_write(u32x4* lds, int g0, int nxg, int nxg_pad,
                                                  const u32x4 (&v)[split_round<F>()])
{
    constexpr int G = Traits<F>::kXGran;
    const int spare = nxg_pad + (threadIdx.x & 63);
#pragma unroll
    for (int k = 0; k < split_round<F>(); ++k) {
        const int g = g0 + k * NT;
        const u32x4 vz = g < nxg ? v[k] : u32x4{0u, 0u, 0u, 0u};
        const int dst = g < nxg_pad ? staged_index<F>(g / G, g % G, nxg_pad / G) : spare;
        lds[dst] = (F == kQ4) ? q4_pair_x(vz) : vz;
    }
}

// ---------------------------------------------------------------- streaming kernel
// Preconditions (checked by the host): N is a multiple of Traits<F>::kElems,
// A and x are 16-byte aligned, M >= 1, and the launch provides
// 4 * stream_lds_words<F, XG>(N / Traits<F>::kElems) bytes of dynamic LDS.
//
// Each wave owns the rows wave_id, wave_id + nwaves, ... and walks them as
// one linear sequence of units; a unit is one pass over a row (one 16-byte
// chunk per lane, 1 KiB per wave).  Loads run D units ahead of the
// arithmetic in straight-line code, so the wait before each unit only needs
// the oldest of D outstanding loads.  The first D loads are issued at
// kernel start (INT4: right after x is staged).  In a ragged last pass
// (fewer than 64 chunks) the lanes past the row end contribute nothing,
// whatever A or x hold (no 0 * inf = NaN from them): FP32/FP16 load chunk 0
// with plain global loads and discard its products; the other formats read A
// through a buffer resource of exactly one row's bytes, which returns zeros
// there, against zero x (zero-padded in LDS, or read through a resource of
// exactly x's bytes).  The unit count is padded to a multiple of D; padded
// units re-read the wave's last row and are never stored.
//
//   XG  x granules are loaded with each unit (through L1/L2) instead of
//       being staged in LDS: no staging and no barrier, at the cost of
//       G x loads per A load.
template <int F, bool XG>
__host__ __device__ constexpr int stream_lds_words(int nchunks)
{
    // 16-byte granules of x for whole passes (zero past the row end)
    return XG ? 0 : ((nchunks + 63) / 64) * 64 * Traits<F>::kXGran * 4;
}

// Buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes
// return zero, which is how lanes past a row's end contribute nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Order of the A prologue and the staging of x (with x in LDS):
//   0  the first D units of A, then the staging (loads, LDS writes);
//   1  the staging, then the first D units of A;
//   2  the first round of staging loads, then the first D units of A, then
//      the round's LDS writes and any further rounds: the first round's loads
//      are the older ones in the wave's in-order load counter, so its LDS
//      writes wait only for them while A is in flight (needs
//      kSplitSpareBytes more LDS than the staged x).
template <int F>
__host__ __device__ constexpr int default_stage_order()
{
    return F == kQ4 ? 1 : 0;
}

template <int F, int WAVES, int D, bool NT, bool XG, int STG = default_stage_order<F>()>
__global__ void __launch_bounds__(WAVES * 64)
gemv_stream(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
            const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    using T = Traits<F>;
    static_assert(WAVES <= 16, "at most 1024 threads per workgroup");
    constexpr int kAux = NT ? 2 : 0;   // buffer-load cache policy: non-temporal
    constexpr int NT_ = WAVES * 64;
    constexpr int G = T::kXGran;       // x granules per unit
    extern __shared__ u32x4 lds_x[];
    const int lane = threadIdx.x & 63;
    const int nchunks = N / T::kElems;
    const int P = (nchunks + 63) >> 6;          // units per row
    const uint32_t row_bytes = (uint32_t)nchunks * 16;
    const int groups = N / 128;                 // INT4 scales per row
    const int wave_id = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = gridDim.x * WAVES;
    const int my_rows = wave_id < M ? (M - 1 - wave_id) / nwaves + 1 : 0;
    const int units = my_rows * P;
    const int units_pad = (units + D - 1) / D * D;
    // a wave without rows (past M) may issue its prologue on row 0 and
    // discard it (split staging, below)
    const int last_row = my_rows > 0 ? wave_id + (my_rows - 1) * nwaves : 0;
    const int nxg = nchunks * G;
    const int nxg_pad = P * 64 * G;             // staged granules, zero past the row end
    const u32x4* xg = reinterpret_cast<const u32x4*>(x);

    // A unit's loads: the row's resource (wave-uniform), the pass offset
    // (wave-uniform) and the lane's fixed offset.  The whole offset goes in
    // the VGPR operand, which is what the range check covers (the SGPR
    // offset stays 0), so lanes past the row end read zeros.
    const int lane_off = lane * 16;
    constexpr int XGR = XG ? G : 1;   // x granules per unit held in registers
    const auto xrsrc = make_rsrc(x, (uint32_t)nxg * 16);   // XG: zeros past x's end
    // FP32/FP16 read A and x with plain global loads (measured faster for
    // them than buffer loads); the others use buffer loads throughout
    constexpr bool kGlobal = XG && (F == kF32 || F == kF16 || F == kF16H);
    u32x4 buf[D];
    u32x4 xbuf[XG ? D : 1][XGR];
    uint16_t sbuf[D];
    int l_row = wave_id, l_pass = 0;
    auto issue = [&](int d) {
        const int row = l_row <= last_row ? l_row : last_row;
        if constexpr (kGlobal) {
            // a lane past the row end loads chunk 0 of A and of x and
            // discards its products (see consume)
            const int c = l_pass * 64 + lane;
            const int cc = c < nchunks ? c : 0;
            buf[d] = load16<NT>(reinterpret_cast<const u32x4*>(A + (int64_t)row * row_bytes) + cc);
            xbuf[d][0] = xg[cc];
        } else {
            const int voff = lane_off + l_pass * 1024;
            const auto rsrc = make_rsrc(A + (int64_t)row * row_bytes, row_bytes);
            buf[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, kAux));
            if constexpr (XG) {
                // granules c*G .. c*G+G-1 of x for chunk c = pass*64 + lane
#pragma unroll
                for (int k = 0; k < XGR; ++k)
                    xbuf[d][k] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, voff * XGR + k * 16, 0, 0));
            }
        }
        if constexpr (F == kQ4) {
            const auto srsrc = make_rsrc(scale + (int64_t)row * groups, (uint32_t)groups * 2);
            sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (lane >> 2) * 2 + l_pass * 32, 0, 0);
        } else if constexpr (F == kQ8) {
            // the row scale travels with every unit of the row, in load order,
            // so the row end needs no load of its own (which would have to
            // wait for every A load in flight)
            sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(scale + row, 2), 0, 0, 0);
        }
        if (++l_pass == P) {
            l_pass = 0;
            l_row += nwaves;
        }
    };

    // With x staged in LDS the order of the prologue and the staging
    // matters (see default_stage_order).
    bool issued = false;
    if ((XG || STG == 0) && units > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            issue(d);
        issued = true;
    }
    if constexpr (!XG) {
        if constexpr (STG == 2) {
            // rounds of SR granules per thread; the A prologue goes
            // out after the first round's loads, so the first round's LDS
            // writes wait only for those older loads while A is in flight
            constexpr int SR = split_round<F>();
            u32x4 v[SR];
            split_round_load<F, NT_>(xg, threadIdx.x, nxg, v);
            // every wave issues the prologue here, without a branch: a branch
            // around it leaves the compiler two paths with different loads in
            // flight, and it then waits for the A loads before the LDS writes
#pragma unroll
            for (int d = 0; d < D; ++d)
                issue(d);
            issued = true;
            split_round_write<F, NT_>(lds_x, threadIdx.x, nxg, nxg_pad, v);
            for (int g0 = threadIdx.x + SR * NT_; g0 - (int)threadIdx.x < nxg_pad; g0 += SR * NT_) {
                split_round_load<F, NT_>(xg, g0, nxg, v);
                split_round_write<F, NT_>(lds_x, g0, nxg, nxg_pad, v);
            }
        } else {
            stage_x<F, NT_>(xg, lds_x, nxg, nxg_pad);
        }
        __syncthreads();
    }
    if (units == 0)
        return;
    if (!issued) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            issue(d);
    }

    float acc = 0.0f;
    f16x2 acch = {(_Float16)0.0f, (_Float16)0.0f};   // FP16 accumulation only
    int c_row = wave_id, c_pass = 0;
    // One unit of arithmetic: a = the unit's 16 bytes of A per lane, xv = its
    // x granules in staged layout (INT4: pair-reordered).
    auto accumulate = [&](u32x4 a, const u32x4 (&xv)[G], uint16_t sraw) {
        if constexpr (F == kF32) {
            acc = chunk_f32(a, xv[0], acc);
        } else if constexpr (F == kF16) {
            acc = chunk_f16(a, xv[0], acc);
        } else if constexpr (F == kF16X32) {
            acc = chunk_f16x32(a, xv[0], xv[1 % G], acc);
        } else if constexpr (F == kF16H) {
            acch = chunk_f16h(a, xv[0], acch);
        } else if constexpr (F == kQ8) {
            acc = q8_chunk(a, xv[0], xv[G - 1], acc);
        } else {
            const u32x4 xp[4] = {xv[0], xv[1 % G], xv[2 % G], xv[3 % G]};
            acc = chunk_q4(a, xp, half_bits_to_float(sraw), acc);
        }
    };
    // Count the unit; at a row's last unit reduce and store.
    auto finish_unit = [&](uint16_t sraw) {
        if (++c_pass == P) {
            if constexpr (F == kF16H) {
                acc = (float)acch.x + (float)acch.y;
                acch = f16x2{(_Float16)0.0f, (_Float16)0.0f};
            }
            float t = wave_sum(acc);
            if (lane == 0 && c_row < M) {
                if constexpr (F == kQ8)
                    t *= half_bits_to_float(sraw);   // this row's scale (see issue)
                y[c_row] = t;
            }
            acc = 0.0f;
            c_pass = 0;
            c_row += nwaves;
        }
    };
    auto consume = [&](int d) {
        const int cc = c_pass * 64 + lane;       // < P * 64: staged (possibly zero) x
        const u32x4 a = buf[d];
        u32x4 xv[G];
        if constexpr (XG) {
#pragma unroll
            for (int k = 0; k < G; ++k)
                xv[k] = (F == kQ4) ? q4_pair_x(xbuf[d][k % XGR]) : xbuf[d][k % XGR];
        } else {
#pragma unroll
            for (int k = 0; k < G; ++k)
                xv[k] = lds_x[staged_index<F>(cc, k, P * 64)];
        }
        if constexpr (kGlobal) {
            // past the row end: keep the sums as they were (one select,
            // cheaper than zeroing A or x)
            const float acc0 = acc;
            const f16x2 acch0 = acch;
            accumulate(a, xv, sbuf[d]);
            if (cc >= nchunks) {
                acc = acc0;
                acch = acch0;
            }
        } else {
            accumulate(a, xv, sbuf[d]);
        }
        finish_unit(sbuf[d]);
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

// ---------------------------------------------------------------- x in registers (rows of K units)
// For rows of exactly K units (K = 1, 2 or 3), lane l's chunks are l, l + 64,
// ... in every row, so each wave loads its lanes' x granules for all K passes
// once, straight into registers (through a resource of x's bytes: zeros past
// the row end), and streams its rows like gemv_stream with no LDS staging
// and no barrier.  With D a multiple of K, load slot d always holds pass
// d % K, so the pass of every unit, and the row end, are known at compile
// time.
//
// Preconditions (checked by the host): ceil(N / kElems / 64) == K,
// D % K == 0, A and x 16-byte aligned, 1 <= M <= 2^30.  No dynamic LDS.
template <int F, int WAVES, int D, int K>
__global__ void __launch_bounds__(WAVES * 64)
gemv_xreg(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
          const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    static_assert(D % K == 0, "load slots must map to fixed passes");
    using T = Traits<F>;
    constexpr int G = T::kXGran;
    const int lane = threadIdx.x & 63;
    const int nchunks = N / T::kElems;
    const uint32_t row_bytes = (uint32_t)nchunks * 16;
    const int groups = N / 128;                 // INT4 scales per row
    const int wave_id = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = gridDim.x * WAVES;
    const int my_rows = wave_id < M ? (M - 1 - wave_id) / nwaves + 1 : 0;
    if (my_rows == 0)
        return;
    const int units = my_rows * K;
    const int units_pad = (units + D - 1) / D * D;
    const int last_row = wave_id + (my_rows - 1) * nwaves;
    constexpr int kAux = 2;                     // A: non-temporal

    const auto xrsrc = make_rsrc(x, (uint32_t)nchunks * G * 16);
    u32x4 xr[K][G];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int g = 0; g < G; ++g)
            xr[k][g] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, ((k * 64 + lane) * G + g) * 16, 0, 0));

    u32x4 buf[D];
    uint16_t sbuf[D];
    int l_row = wave_id;
    auto issue = [&](int d) {
        const int pass = d % K;
        const int row = l_row <= last_row ? l_row : last_row;
        const auto rsrc = make_rsrc(A + (int64_t)row * row_bytes, row_bytes);
        buf[d] = __builtin_bit_cast(u32x4,
                                    __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane * 16 + pass * 1024, 0, kAux));
        if constexpr (F == kQ4) {
            const auto srsrc = make_rsrc(scale + (int64_t)row * groups, (uint32_t)groups * 2);
            sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (lane >> 2) * 2 + pass * 32, 0, 0);
        } else if constexpr (F == kQ8) {
            sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(scale + row, 2), 0, 0, 0);
        }
        if (pass == K - 1)
            l_row += nwaves;
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        issue(d);

    // x is older than every A load in the counter: ready before the first unit
    if constexpr (F == kQ4) {
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int g = 0; g < G; ++g)
                xr[k][g] = q4_pair_x(xr[k][g]);
    }

    float acc = 0.0f;
    f16x2 acch = {(_Float16)0.0f, (_Float16)0.0f};   // FP16 accumulation only
    int c_row = wave_id;
    auto consume = [&](int d) {
        const int pass = d % K;
        if constexpr (F == kF32) {
            acc = chunk_f32(buf[d], xr[pass][0], acc);
        } else if constexpr (F == kF16) {
            acc = chunk_f16(buf[d], xr[pass][0], acc);
        } else if constexpr (F == kF16X32) {
            acc = chunk_f16x32(buf[d], xr[pass][0], xr[pass][G - 1], acc);
        } else if constexpr (F == kF16H) {
            acch = chunk_f16h(buf[d], xr[pass][0], acch);
        } else if constexpr (F == kQ8) {
            acc = q8_chunk(buf[d], xr[pass][0], xr[pass][G - 1], acc);
        } else {
            acc = chunk_q4(buf[d], xr[pass], half_bits_to_float(sbuf[d]), acc);
        }
        if (pass == K - 1) {
            if constexpr (F == kF16H) {
                acc = (float)acch.x + (float)acch.y;
                acch = f16x2{(_Float16)0.0f, (_Float16)0.0f};
            }
            float t = wave_sum(acc);
            if (lane == 0 && c_row < M) {
                if constexpr (F == kQ8)
                    t *= half_bits_to_float(sbuf[d]);
                y[c_row] = t;
            }
            acc = 0.0f;
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

// ---------------------------------------------------------------- packed short rows (INT8/INT4)
// Rows shorter than half a wave load (at most 32 chunks): a wave load takes
// R = 64 / L rows at once, L = the power of two >= the chunk count, and
// lane l works on chunk l % L of row g * R + l / L of row group g.  A lane's
// chunk, and so its x, is the same in every group: each wave loads its
// lanes' x granules once, straight into registers (no LDS, no barrier).
// Each group's partial sums meet in a segmented butterfly of L lanes.
// Groups stream D ahead as in gemv_stream.
//
// Preconditions (checked by the host): F is kQ8 or kQ4, 1 <= N / kElems <= 32,
// A and x 16-byte aligned, 1 <= M <= 2^30 (row and group indices stay in
// int).  No dynamic LDS.
template <int F>
__host__ __device__ constexpr int packed_lanes(int nchunks)
{
    int L = 1;
    while (L < nchunks)
        L <<= 1;
    return L;
}

// Sum over aligned groups of L lanes (L a power of two, at most 32); the
// result is valid in every lane of the group.
__device__ __forceinline__ float segment_sum(float v, int L)
{
    if (L >= 2)
        v += dpp_mov<0xB1>(v);   // lane ^ 1
    if (L >= 4)
        v += dpp_mov<0x4E>(v);   // lane ^ 2
    if (L >= 8)
        v += dpp_mov<0x141>(v);  // other quad of the 8-lane half row
    if (L >= 16)
        v += dpp_mov<0x140>(v);  // other half of the 16-lane row
    if (L >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    return v;
}

template <int F, int WAVES, int D>
__global__ void __launch_bounds__(WAVES * 64)
gemv_packed(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
            const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    static_assert(F == kQ8 || F == kQ4, "packed short rows: INT8/INT4 only");
    using T = Traits<F>;
    constexpr int G = T::kXGran;
    const int lane = threadIdx.x & 63;
    const int nchunks = N / T::kElems;
    const int L = packed_lanes<F>(nchunks);
    const int R = 64 / L;
    const int sub = lane / L;                    // row within the group
    const int c = lane & (L - 1);                // this lane's chunk
    const uint32_t row_bytes = (uint32_t)nchunks * 16;
    const int sgroups = N / 128;                 // INT4 scales per row
    const int groups = (M + R - 1) / R;
    const int wave_id = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = gridDim.x * WAVES;
    const int mine = wave_id < groups ? (groups - 1 - wave_id) / nwaves + 1 : 0;
    const int mine_pad = (mine + D - 1) / D * D;
    const int last = wave_id + (mine - 1) * nwaves;
    if (mine == 0)
        return;
    // x: this lane's chunk, G granules, straight into registers through a
    // resource of exactly x's bytes (zeros for lanes past the row end); no
    // LDS and no barrier.
    const auto xrsrc = make_rsrc(x, (uint32_t)nchunks * G * 16);
    u32x4 xv[G];
#pragma unroll
    for (int k = 0; k < G; ++k)
        xv[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (c * G + k) * 16, 0, 0));

    // One resource per row group (wave-uniform, so the loads need no
    // per-lane descriptors) covering the group's rows below M; a lane's
    // offset selects its row and chunk.  Lanes past the row end get an
    // offset beyond every range and so read zeros, as do rows past M.
    constexpr uint32_t kOutside = 0x7FFFFFF0u;
    const bool live = c < nchunks;
    const uint32_t a_off = live ? (uint32_t)sub * row_bytes + (uint32_t)c * 16 : kOutside;
    const uint32_t s_off = live ? (uint32_t)(F == kQ4 ? sub * sgroups + (c >> 2) : sub) * 2 : kOutside;
    u32x4 buf[D];
    uint16_t sbuf[D];
    int l_g = wave_id;
    auto issue = [&](int d) {
        const int g = l_g <= last ? l_g : last;
        const int r0 = g * R;
        const uint32_t nrows = (uint32_t)(M - r0 < R ? M - r0 : R);
        const auto rsrc = make_rsrc(A + (int64_t)r0 * row_bytes, nrows * row_bytes);
        buf[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, a_off, 0, 2));
        const uint32_t srow = F == kQ4 ? (uint32_t)sgroups : 1u;
        const auto srsrc = make_rsrc(scale + (int64_t)r0 * srow, nrows * srow * 2);
        sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, s_off, 0, 0);
        l_g += nwaves;
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        issue(d);
    // x arrives before the first A loads (older in the load counter)
    if constexpr (F == kQ4) {
#pragma unroll
        for (int k = 0; k < G; ++k)
            xv[k] = q4_pair_x(xv[k]);
    }

    int c_g = wave_id;
    auto consume = [&](int d) {
        float acc;
        if constexpr (F == kQ4) {
            acc = chunk_q4(buf[d], xv, half_bits_to_float(sbuf[d]), 0.0f);
        } else {
            acc = q8_chunk(buf[d], xv[0], xv[G - 1], 0.0f);
        }
        float t = segment_sum(acc, L);
        if (c == 0 && c_g <= last && c_g * R + sub < M) {
            const int row = c_g * R + sub;
            if constexpr (F == kQ8)
                t *= half_bits_to_float(sbuf[d]);
            y[row] = t;
        }
        c_g += nwaves;
    };
    for (int k0 = D; k0 < mine_pad; k0 += D) {
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

// ---------------------------------------------------------------- split rows (few, long rows)
// When the rows are too few for one wave per row to fill the chip, a
// workgroup of S waves takes one row: wave w streams the row's units w,
// w + S, w + 2S, ... (one 16-byte chunk per lane and unit, as in
// gemv_stream), D in flight; each wave reduces its 64 lane sums, the S wave
// sums meet in LDS, and the first thread adds them in wave order and stores
// y.  x is read with each unit through the caches (as gemv_stream's XG
// form): the S waves of a row read disjoint parts of it.  The cross-wave step
// is the LDS reduction of a row that spans waves ("membound", the llama.cpp
// walkthrough's block-per-row kernel, and "cuda-gemv-optimization", the
// shared-memory kernel: partial sums of one row meet in shared memory).
//
// Preconditions (checked by the host): N is a multiple of Traits<F>::kElems,
// A and x are 16-byte aligned, 1 <= S <= units per row, the grid has one
// workgroup per row (M <= 2^30 / (S * 64)).
template <int F, int S, int D>
__global__ void __launch_bounds__(S * 64)
gemv_split(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
           const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    static_assert(F != kF16H, "FP16 accumulation keeps one wave per row");
    using T = Traits<F>;
    constexpr int G = T::kXGran;
    constexpr bool kGlobal = F == kF32 || F == kF16;   // as gemv_stream: plain global loads
    __shared__ float part[S];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x;
    if (row >= M)   // the whole workgroup: the grid has one workgroup per row
        return;
    const int nchunks = N / T::kElems;
    const int P = (nchunks + 63) >> 6;
    const int units = (P - w + S - 1) / S;      // passes w, w + S, ... < P (at least 1)
    const int units_pad = (units + D - 1) / D * D;
    const uint32_t row_bytes = (uint32_t)nchunks * 16;
    const int groups = N / 128;                 // INT4 scales per row
    const u32x4* xg = reinterpret_cast<const u32x4*>(x);
    const uint8_t* arow = A + (int64_t)row * row_bytes;
    const auto arsrc = make_rsrc(arow, row_bytes);
    const auto xrsrc = make_rsrc(x, (uint32_t)nchunks * G * 16);
    const auto srsrc = make_rsrc(scale + (int64_t)row * groups, (uint32_t)groups * 2);
    constexpr int kAux = 2;                     // A: non-temporal

    u32x4 buf[D];
    u32x4 xbuf[D][G];
    uint16_t sbuf[D];
    // unit j (padded units re-read the wave's last unit and are not added)
    auto issue = [&](int d, int j) {
        const int pass = w + S * (j < units ? j : units - 1);
        if constexpr (kGlobal) {
            const int c = pass * 64 + lane;
            const int cc = c < nchunks ? c : 0;
            buf[d] = load16<true>(reinterpret_cast<const u32x4*>(arow) + cc);
            xbuf[d][0] = xg[cc];
        } else {
            const int voff = lane * 16 + pass * 1024;
            buf[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, voff, 0, kAux));
#pragma unroll
            for (int k = 0; k < G; ++k)
                xbuf[d][k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, voff * G + k * 16, 0, 0));
        }
        if constexpr (F == kQ4)
            sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (lane >> 2) * 2 + pass * 32, 0, 0);
        else
            sbuf[d] = 0;
    };
    float acc = 0.0f;
    auto consume = [&](int d, int j) {
        const int pass = w + S * (j < units ? j : units - 1);
        const int cc = pass * 64 + lane;
        const u32x4 a = buf[d];
        u32x4 xv[G];
#pragma unroll
        for (int k = 0; k < G; ++k)
            xv[k] = (F == kQ4) ? q4_pair_x(xbuf[d][k]) : xbuf[d][k];
        float t = acc;
        if constexpr (F == kF32) {
            t = chunk_f32(a, xv[0], t);
        } else if constexpr (F == kF16) {
            t = chunk_f16(a, xv[0], t);
        } else if constexpr (F == kF16X32) {
            t = chunk_f16x32(a, xv[0], xv[G - 1], t);
        } else if constexpr (F == kQ8) {
            t = q8_chunk(a, xv[0], xv[G - 1], t);
        } else {
            const u32x4 xp[4] = {xv[0], xv[1 % G], xv[2 % G], xv[3 % G]};
            t = chunk_q4(a, xp, half_bits_to_float(sbuf[d]), t);
        }
        // a padded unit, or (global loads) a lane past the row end, adds nothing
        const bool live = j < units && (!kGlobal || cc < nchunks);
        acc = live ? t : acc;
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        issue(d, d);
    for (int j0 = D; j0 < units_pad; j0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            consume(d, j0 - D + d);
            issue(d, j0 + d);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        consume(d, units_pad - D + d);

    const float t = wave_sum(acc);
    if (lane == 0)
        part[w] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        float sum = part[0];
#pragma unroll
        for (int k = 1; k < S; ++k)
            sum += part[k];
        if constexpr (F == kQ8)
            sum *= half_bits_to_float(scale[row]);
        y[row] = sum;
    }
}

// ---------------------------------------------------------------- row slabs, x slices in registers
// Sums of eight values over the 64 lanes at once: on return lane l holds the
// sum of v[l >> 3].  A butterfly that halves the values at each step instead
// of reducing each one separately: v_permlane32_swap pairs v[i] with v[i+4]
// across the wave's halves (lanes 0-31 keep rows 0-3, lanes 32-63 rows 4-7),
// v_permlane16_swap pairs the remaining values across 16-lane rows, a select
// and a DPP rotation by 8 across half rows, then three DPP adds within each
// 8-lane group: 18 instructions for eight sums, where eight wave_sum calls
// take about 70.
__device__ __forceinline__ float wave_sum8(const float (&v)[8])
{
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[i]),
                                                        __builtin_bit_cast(unsigned, v[i + 4]), false, false);
        b[i] = as_f(p[0]) + as_f(p[1]);
    }
    float c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, b[i]),
                                                        __builtin_bit_cast(unsigned, b[i + 2]), false, false);
        c[i] = as_f(p[0]) + as_f(p[1]);
    }
    // c[0] holds rows 0, 2, 4, 6 and c[1] rows 1, 3, 5, 7 in the four 16-lane
    // rows; lanes with bit 3 set keep c[1]
    const bool odd = (threadIdx.x & 8) != 0;
    const float keep = odd ? c[1] : c[0];
    const float give = odd ? c[0] : c[1];
    float r = keep + dpp_mov<0x128>(give);   // row_ror:8: the other half row
    r += dpp_mov<0xB1>(r);    // lane ^ 1
    r += dpp_mov<0x4E>(r);    // lane ^ 2
    r += dpp_mov<0x141>(r);   // row_half_mirror: the other quad
    return r;
}

// The same for four values: on return lane l holds the sum of v[l >> 4]
// (10 instructions).
__device__ __forceinline__ float wave_sum4(const float (&v)[4])
{
    float b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[i]),
                                                        __builtin_bit_cast(unsigned, v[i + 2]), false, false);
        b[i] = as_f(p[0]) + as_f(p[1]);
    }
    // b[0] holds rows 0 and 2, b[1] rows 1 and 3 in the wave's halves
    const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, b[0]),
                                                    __builtin_bit_cast(unsigned, b[1]), false, false);
    float r = as_f(p[0]) + as_f(p[1]);
    r += dpp_mov<0x128>(r);   // row_ror:8: the other half row
    r += dpp_mov<0xB1>(r);    // lane ^ 1
    r += dpp_mov<0x4E>(r);    // lane ^ 2
    r += dpp_mov<0x141>(r);   // row_half_mirror: the other quad
    return r;
}

// Long INT8/INT4 and FP16-with-FP32-x rows, whose x every workgroup of
// gemv_stream would stage in LDS: a workgroup of S waves takes R = 4 or 8
// consecutive rows (a slab) at a time, and wave w owns the passes w, w + S, ...,
// w + (Q - 1) S of every row of the slab (S * Q = P units per row).  Lane l's
// chunks are then the same in every row, so each wave loads its lanes' x for
// its Q passes into registers once (as gemv_xreg does for a whole row) and
// streams the slab's R Q units, D in flight, into one FP32 sum per row, with
// no x staging and no LDS read of x.  The wave then reduces its R row sums
// at once (wave_sum8, wave_sum4) and leaves them in LDS; the slab's first R threads
// add the S wave sums of their row in wave order (deterministic) and store
// y: the cross-wave step of a row that spans waves, as in gemv_split, once
// per slab.  Units past the slab's last row are padding: they re-read that
// row's units and are not stored.
//
// Preconditions (checked by the host): F is kQ8, kQ4 or kF16X32; the row is
// P = ceil(N / kElems / 64) = S * Q units with blockDim.x = 64 S, S <= 16;
// A and x 16-byte aligned; 1 <= M <= 2^30.  No dynamic LDS.
template <int F, int Q, int D, int kSlabRows>
__global__ void __launch_bounds__(1024)
gemv_slab(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
          const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    static_assert(F == kQ8 || F == kQ4 || F == kF16X32, "formats that would stage x");
    static_assert(kSlabRows == 4 || kSlabRows == 8, "rows per slab");
    static_assert((kSlabRows * Q) % D == 0 && D % Q == 0, "load slots must map to fixed rows and passes");
    using T = Traits<F>;
    constexpr int G = T::kXGran;
    constexpr int U = kSlabRows * Q;            // units per wave and slab
    constexpr int kAux = 2;                     // A: non-temporal
    __shared__ float part[16 * kSlabRows];      // [wave][row of the slab]
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int nchunks = N / T::kElems;
    const uint32_t row_bytes = (uint32_t)nchunks * 16;
    const int groups = N / 128;                 // INT4 scales per row
    const int nslabs = (M + kSlabRows - 1) / kSlabRows;

    // this lane's x granules for passes w + q S (zeros past the row end)
    const auto xrsrc = make_rsrc(x, (uint32_t)nchunks * G * 16);
    u32x4 xr[Q][G];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int g = 0; g < G; ++g)
            xr[q][g] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (((w + q * S) * 64 + lane) * G + g) * 16, 0, 0));
    bool paired = false;   // INT4: x reordered for q4_word once, after the first A loads

    for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
        const int row0 = slab * kSlabRows;
        const int rows = M - row0 < kSlabRows ? M - row0 : kSlabRows;
        // INT8: the slab's row scales, one per thread of the first 8 (zeros
        // past the slab), loaded before A so that they are the oldest loads
        float srow = 0.0f;
        if constexpr (F == kQ8)
            srow = half_bits_to_float(__builtin_amdgcn_raw_buffer_load_b16(
                make_rsrc(scale + row0, (uint32_t)rows * 2), (int)threadIdx.x * 2, 0, 0));

        u32x4 buf[D];
        uint16_t sbuf[D];
        // unit j: slab row j / Q (padding re-reads the last row), pass w + (j % Q) S
        auto issue = [&](int d, int j) {
            const int r = j / Q;
            const int row = row0 + (r < rows ? r : rows - 1);
            const int pass = w + (j % Q) * S;
            const auto rsrc = make_rsrc(A + (int64_t)row * row_bytes, row_bytes);
            buf[d] = __builtin_bit_cast(u32x4,
                                        __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane * 16 + pass * 1024, 0, kAux));
            if constexpr (F == kQ4) {
                const auto srsrc = make_rsrc(scale + (int64_t)row * groups, (uint32_t)groups * 2);
                sbuf[d] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (lane >> 2) * 2 + pass * 32, 0, 0);
            } else {
                sbuf[d] = 0;
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d)
            issue(d, d);
        if constexpr (F == kQ4) {
            // x is older than every A load in the counter
            if (!paired) {
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        xr[q][g] = q4_pair_x(xr[q][g]);
                paired = true;
            }
        }

        float acc[kSlabRows];
#pragma unroll
        for (int r = 0; r < kSlabRows; ++r)
            acc[r] = 0.0f;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int d = j % D, q = j % Q, r = j / Q;
            if constexpr (F == kF16X32)
                acc[r] = chunk_f16x32(buf[d], xr[q][0], xr[q][G - 1], acc[r]);
            else if constexpr (F == kQ8)
                acc[r] = q8_chunk(buf[d], xr[q][0], xr[q][G - 1], acc[r]);
            else
                acc[r] = chunk_q4(buf[d], xr[q], half_bits_to_float(sbuf[d]), acc[r]);
            if (j + D < U)
                issue(d, j + D);
        }
        // lane l holds row l / (64 / R)
        constexpr int kShift = kSlabRows == 8 ? 3 : 4;
        float t;
        if constexpr (kSlabRows == 8)
            t = wave_sum8(acc);
        else
            t = wave_sum4(acc);
        if ((lane & ((1 << kShift) - 1)) == 0 && (lane >> kShift) < rows)
            part[w * kSlabRows + (lane >> kShift)] = t;

        __syncthreads();
        if ((int)threadIdx.x < rows) {
            float sum = part[threadIdx.x];
            for (int k = 1; k < S; ++k)
                sum += part[k * kSlabRows + threadIdx.x];
            if constexpr (F == kQ8)
                sum *= srow;
            y[row0 + threadIdx.x] = sum;
        }
        __syncthreads();   // part is reused by the next slab
    }
}

// ---------------------------------------------------------------- element-wise kernel
// Any N >= 0 and any alignment: one wave per row, lane l takes columns
// l, l+64, ... with scalar loads (INT4: bytes l, l+64, ..., two columns
// each), the loops unrolled so that several loads are in flight (the sums
// keep their order).  Four waves per workgroup; waves walk rows
// 4 x gridDim.x apart.
template <int F>
__global__ void __launch_bounds__(256)
gemv_elementwise(const uint8_t* __restrict__ A, const uint16_t* __restrict__ scale,
                 const uint8_t* __restrict__ x, float* __restrict__ y, int M, int N)
{
    const int lane = threadIdx.x & 63;
    // rows walked grid-stride (wave-uniform), so any grid covers them
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < M; row += stride) {
        float acc = 0.0f;
        if constexpr (F == kF32) {
            const float* a = reinterpret_cast<const float*>(A) + (int64_t)row * N;
            const float* xf = reinterpret_cast<const float*>(x);
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                acc = __builtin_fmaf(a[j], xf[j], acc);
        } else if constexpr (F == kF16) {
            const uint16_t* a = reinterpret_cast<const uint16_t*>(A) + (int64_t)row * N;
            const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                acc = __builtin_fmaf(half_bits_to_float(a[j]), half_bits_to_float(xh[j]), acc);
        } else if constexpr (F == kF16X32) {
            const uint16_t* a = reinterpret_cast<const uint16_t*>(A) + (int64_t)row * N;
            const float* xf = reinterpret_cast<const float*>(x);
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                acc = __builtin_fmaf(half_bits_to_float(a[j]), xf[j], acc);
        } else if constexpr (F == kF16H) {
            // one binary16 running sum per lane (ceil(N/64) terms)
            const _Float16* a = reinterpret_cast<const _Float16*>(A) + (int64_t)row * N;
            const _Float16* xh = reinterpret_cast<const _Float16*>(x);
            _Float16 h = (_Float16)0.0f;
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                h = __builtin_fmaf16(a[j], xh[j], h);
            acc = (float)h;
        } else if constexpr (F == kQ8) {
            const int8_t* a = reinterpret_cast<const int8_t*>(A) + (int64_t)row * N;
            const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
#pragma unroll 8
            for (int64_t j = lane; j < N; j += 64)
                acc = __builtin_fmaf((float)a[j], half_bits_to_float(xh[j]), acc);
        } else {
            const int half_n = N / 2;
            const uint8_t* a = A + (int64_t)row * half_n;
            const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
            const uint16_t* srow = scale + (int64_t)row * (N / 128);
#pragma unroll 4
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
