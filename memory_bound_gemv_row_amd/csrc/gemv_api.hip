// gemv_api.hip -- C ABI of the gfx950 GEMV library (declared in include/gemv.h).
//
// Host side only: argument validation, choice of kernel variant and launch
// geometry, and the launch itself on the caller's stream.  The host
// launcher of the pages picks the grid and block and launches
// asynchronously ("Making GEMV Fast", the launch_kernel functions); here the
// grid is sized from the row count and the device's compute-unit count, and
// a launch failure is returned as a status instead of ending the process.
#include "gemv.h"
#include "device_info.hpp"
#include "gemv_kernels.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

namespace gemv {
namespace {

// Staged x up to this size takes the plans tuned for ordinary rows; longer
// rows have their own plans, up to the LDS one workgroup may hold.
constexpr int kLdsBytes = 64 * 1024;
constexpr bool kNT = true;             // stream A with non-temporal loads
using gemv_device::Device;

int elems_per_chunk(int kind)
{
    switch (kind) {
    case kF32: return Traits<kF32>::kElems;
    case kF16: return Traits<kF16>::kElems;
    case kQ8: return Traits<kQ8>::kElems;
    case kF16X32: return Traits<kF16X32>::kElems;
    case kF16H: return Traits<kF16H>::kElems;
    default: return Traits<kQ4>::kElems;
    }
}

// Bytes of x one workgroup stages (whole passes, zero past the row end),
// in 64 bits: rows near 2^30 elements would overflow an int.  FP32/FP16 (either
// accumulation) read x with each unit and stage nothing.
int64_t lds_bytes(int kind, int nchunks)
{
    int64_t granules = 0;   // 16-byte granules of x per chunk
    switch (kind) {
    case kQ8: granules = Traits<kQ8>::kXGran; break;
    case kQ4: granules = Traits<kQ4>::kXGran; break;
    case kF16X32: granules = Traits<kF16X32>::kXGran; break;
    default: break;
    }
    return ((int64_t)nchunks + 63) / 64 * 64 * granules * 16;
}

// Packed short rows: INT8/INT4 rows of at most this many chunks share wave
// loads; 64 / L rows per load, L the power of two at or above the chunk count.
constexpr int kPackedMaxChunks = 32;

int packed_rows_per_load(int nchunks) { return 64 / packed_lanes<kQ8>(nchunks); }

struct Plan {
    int variant;   // 1 stream + LDS x, 2 stream + global x, 3 element-wise,
                   // 4 packed short rows (INT8/INT4), 5 x in registers,
                   // 6 split rows (several waves per row),
                   // 7 row slabs (INT8/INT4/FP16 with FP32 x: waves own
                   // passes, x slices in registers)
    int grid;
    int block;
    int waves;     // per workgroup
    int rows;      // rows per wave (upper bound); variant 4: row groups per wave;
                   // variant 7: rows per slab (R)
    int D;         // units in flight per wave
    int lds;
    int stg;       // order of A prologue and x staging (default_stage_order)
    int cap;       // at most cap workgroups per CU (0: no cap)
    int xk;        // variant 5: units per row (K); variant 6: waves per row (S);
                   // variant 7: passes per wave (Q)
};

// Split rows (variant 6), chosen after the one-wave-per-row plan p0: where
// p0 leaves the CUs short of waves (fewer than 4 per CU for FP32/FP16, 8
// for FP32/FP16 rows of 16 units and more, 2 for INT4) and the rows are at
// least 4 units long (INT4: at most 16,
// whose x, read with each unit, is four times the bytes of its A), S waves
// share each row, S the least power of two that gives every CU
// kSplitWavesPerCu waves (at most 16, and at least two units per wave);
// each wave streams ceil(P / S) units, 2 or 4 in flight.
// Graph-timed A/B against p0: FP16 64x65536 25.07 -> 6.16 us, INT8
// 16x131072 37.79 -> 8.23, FP32 408x14592 13.29 -> 6.68, FP32 2246x19200
// 43.04 -> 29.95, FP16 278x16896 8.34 -> 5.42, FP16 1024x14336
// 7.89 -> 6.79, INT8 560x6656 4.02 -> 3.00, INT4 363x8704 4.08 -> 3.32;
// where p0 already fills the CUs it won (FP16 1792x4096 4.09 vs 4.19,
// FP32 1024x1024 2.52 vs 2.66, FP16 1024x4096 3.09 vs 3.29), and INT4 rows
// of 18 units lost to it by 60 %.  INT8 and FP16 with FP32 x have rules of
// their own (below), which the brute-force search measured.
// INT8 (since its exact decode) splits up to 6 rows per CU, with S for 4
// waves per CU and 2 units in flight: brute force over every plan on 17
// such shapes put this 1.7 % from the fastest (geometric mean; 8 % at
// worst), the rule above 10.5 % (24 %): INT8 1069x10368 5.61 -> 4.64 us,
// 1453x4224 4.53 -> 3.88, 486x38592 7.97 -> 6.42.
constexpr int kSplitWavesPerCu = 16;

bool split_plan(int kind, int M, int P, int cus, const Plan& p0, Plan* p)
{
    if (kind == kF16H || P < 4 || p0.variant == 3)
        return false;
    int64_t target = (int64_t)kSplitWavesPerCu * cus;
    int depth = 0;   // 0: 2 for two units per wave, else 4
    if (kind == kQ8) {
        if (M > 6 * cus)
            return false;
        target = 4 * (int64_t)cus;
        depth = 2;
    } else if (kind == kF16X32) {
        // up to 7 rows per CU (rows of 16 units and more: 5, above which
        // staged x measured up to 26 % faster: 1702 x 23168 19.79 -> 15.05
        // us), two waves per row (the fewest), 4 in flight below 3 rows per
        // CU, else 2 (512 x 25984: 9.67 us at 2 in flight, 7.42 at 4; 800 x
        // 16384: 7.15 at 2, 7.75 at 4),
        // where S for 16 waves per CU was up to 31 % from the
        // fastest plan (1492 x 5120 6.26 -> 5.11 us, 410 x 24448 7.80 ->
        // 6.74, 977 x 27392 15.19 -> 11.92)
        if (M > (P < 16 ? 7 : 5) * cus)
            return false;
        if (M >= cus)
            target = 0;   // (below one row per CU: enough waves to fill the chip)
        depth = M < 3 * cus ? 4 : 2;
    } else {
        // FP32/FP16 rows of 16 units and more up to 8 waves per CU (x is
        // one granule per unit); otherwise 4, INT4 2 (x per unit is four
        // granules)
        const bool fp = kind == kF32 || kind == kF16;
        const int per_cu = fp && P >= 16 ? 8 : (kind == kQ4 ? 2 : 4);
        if ((int64_t)p0.grid * p0.waves >= (int64_t)per_cu * cus || (kind == kQ4 && P > 16))
            return false;
        if (fp && M >= 2 * cus) {
            // FP32/FP16 from two rows per CU: two waves per row, 4 in flight
            // below 4 rows per CU, else 2 (with the cost model after it,
            // 144 random shapes put the picks 3.5 % (FP32) and 2.9 % (FP16)
            // from the fastest plan, against 3.9 % and 3.4 % with S for 16
            // waves per CU: FP16 696 x 9600 5.27 -> 4.51 us, FP32 686 x 4864
            // 5.17 -> 4.49; 2 in flight from 4 rows per CU: FP32 1345 x
            // 9344 11.20 -> 9.70)
            target = 0;
            depth = M < 4 * cus ? 4 : 2;
        }
    }
    int S = 2;   // P >= 4: two units per wave at least
    while (S < 16 && 4 * S <= P && (int64_t)M * S < target)
        S *= 2;
    const int per_wave = (P + S - 1) / S;
    *p = Plan{};
    p->variant = 6;
    p->xk = S;
    p->waves = S;
    p->block = S * 64;
    p->D = depth > 0 ? depth : (per_wave == 2 ? 2 : 4);   // at least two units per wave
    p->rows = 1;
    p->stg = -1;
    p->lds = 0;
    p->grid = M;
    return true;
}

// Units in flight (4 or 8) and rows per wave (1 or 2) for rows of P units
// (4 <= P < 24) read with x per unit, one row per wave otherwise: a wave
// streams its rows' units as one sequence padded to a multiple of D, and
// the padding re-reads units (a row of 12 units at 8 in flight streams 16:
// FP16 8192x6144 19.9 us against 15.9 without padding).  The choice with
// the least padding wins; ties go to 4 in flight and one row for rows under
// 8 units (more waves), to 8 in flight otherwise.  Two rows per wave only
// where the halved grid still gives every CU a workgroup (two_rows_fill).
void least_padding(int P, bool two_rows_fill, int* D, int* rows)
{
    static constexpr int kShort[4][2] = {{4, 1}, {4, 2}, {8, 1}, {8, 2}};
    static constexpr int kLong[4][2] = {{8, 1}, {8, 2}, {4, 1}, {4, 2}};
    const auto& order = P < 8 ? kShort : kLong;
    int best = 0;
    int64_t best_pad = -1, best_len = 1;
    for (int k = 0; k < 4; ++k) {
        if (order[k][1] == 2 && !two_rows_fill)
            continue;
        const int d = order[k][0], len = order[k][1] * P;
        const int64_t pad = (len + d - 1) / d * d - len;
        // pad / len < best_pad / best_len, compared without division
        if (best_pad < 0 || pad * best_len < best_pad * len) {
            best = k;
            best_pad = pad;
            best_len = len;
        }
    }
    *D = order[best][0];
    *rows = order[best][1];
}

// Whether M rows at two per wave, `waves` waves per workgroup, still give
// each of `cus` CUs a workgroup.
bool two_rows_fill(int64_t M, int waves, int cus)
{
    return (M + 2 * waves - 1) / (2 * waves) >= cus;
}

// Workgroup size and grid of a plan whose waves walk rows: enough waves for
// M rows at p->rows per wave, at most p->cap workgroups per CU (none: 0),
// and at most 2^30 work-items.
void finish_rows(int M, int cus, Plan* p)
{
    p->block = p->waves * 64;
    const int64_t waves_needed = ((int64_t)M + p->rows - 1) / p->rows;
    int64_t grid = (waves_needed + p->waves - 1) / p->waves;
    if (p->cap > 0 && grid > (int64_t)p->cap * cus)
        grid = (int64_t)p->cap * cus;
    p->grid = gemv_device::capped_grid(grid, p->block);
}

// Geometry for one call, chosen from sweeps on MI355X.  A row of nchunks
// 16-byte chunks is P = ceil(nchunks / 64) units (one 1-KiB wave load each).
//   FP32/FP16 (either accumulation), other rows: x read with each unit;
//     rows of 4-23 units: 4 or 8 in flight and one or two rows per wave,
//     whichever pads each wave's stream least (least_padding); rows
//     of 24 units and more: 4 waves, 8 in flight and two rows per wave up to
//     12 rows per CU, 8 in flight and one row per wave (two if the units
//     are not a multiple of 8) from 24 rows per CU or for rows of a
//     multiple of 16 units, two rows and 4 in flight otherwise; one-unit
//     rows (beyond 32 rows per CU) put 4 rows on
//     each wave so that 4 units are in flight without padding.
//   Rows of one unit (any format; FP32/FP16 only up to 32 rows per CU), of
//     two units (FP32/FP16; INT4 up to 16 rows per CU; FP16 with FP32 x
//     beyond that) and of three: x in registers (gemv_xreg), no staging.
//     One-unit rows: 4 waves (8 for FP32/FP16), one unit in flight up to 32
//     rows per CU; up to 64, 4 waves with two rows each, both in flight;
//     beyond that 8 waves, 2 in flight, at most 3 workgroups per CU;
//     two-unit rows 4 waves, 2 in flight (FP16 with FP32 x: at most 6
//     workgroups per CU).  Rows of three units (FP32/FP16, FP16 with FP32 x;
//     INT4 up to 8 rows per CU): 3 in flight, 8 waves (FP32/FP16 beyond 32
//     rows per CU: 4; FP16 with FP32 x: 4 up to 16 rows per CU, beyond
//     that 8 with at most 3 workgroups per CU).
//   INT8, other rows: few rows (M <= 16 x CUs for rows of 2 units, M <= 8 x
//     CUs for rows up to 16 units, save rows of 8 units or more with M <= 4
//     x CUs, which stage x as below with 8 waves, x before A, one workgroup
//     per CU): x read with each unit, 8 waves, 2 (two-unit rows) or 4 in
//     flight -- the staging and its barrier would dominate such launches.
//     Otherwise x is staged: rows of 8 units or more: 4 waves, 4 in flight,
//     split staging (staging loads, A prologue, LDS writes), two rows per
//     wave for rows of 8-10 units where every CU still gets a workgroup,
//     else one row and at most 2 workgroups per CU; rows of 2 units: 8
//     waves, 2 in flight, split staging, at most 3 workgroups per CU; rows
//     of 3-5 units: 4 waves, split staging, at most 3 workgroups per CU;
//     rows of 6 or 7: 8 waves, A first, at most 2 workgroups per CU.  (Up
//     to 6 rows per CU, rows of 4 units and more split instead: split_plan.)
//     Staged x past 64 KiB (rows of 32 units and more): with two workgroups
//     per CU fitting the device's LDS and over 4 x CUs rows, 4 waves, split
//     staging, at most 2 workgroups per CU; otherwise 8 waves, x staged
//     before A, one workgroup per CU -- but x read with each unit (4 waves
//     of two rows, 8 in flight) where only one workgroup fits and M <= 8 x
//     CUs, or where the staged x would not fit at all.
//   INT4, other rows, x staged: rows under 4 units: 8 waves, 2 in flight,
//     split staging, at most 4 workgroups per CU; longer rows: 4 in flight,
//     x staged before A, 4 waves and at most 3 workgroups per CU -- but 8
//     waves and at most 2 for rows of 14-16 units (fewer stagings of x:
//     8192 x 28672 26.0 -> 22.3 us, 4096 x 28672 16.4 -> 13.5; shorter rows
//     gained at some row counts and lost at others).  Staged x past 64 KiB
//     (rows over 16 units): 8 waves, 4 in flight, x staged before A, one
//     workgroup per CU.  x read with each unit (4 waves, 4 in flight)
//     instead for M <= 4 x CUs (any row length), or where the staged x
//     would not fit the device's LDS.
//   INT8/INT4 rows of at most 32 chunks (half a wave load): the packed
//     kernel, 64 / L rows per wave load, 8 waves; with up to 16 row groups
//     per CU one group per wave, beyond that two (both in flight).
//   FP16 with FP32 x: x is twice the bytes of FP16 x, and reading it with
//     every unit costs more cache bandwidth than staging it, once the staging
//     (4N bytes per workgroup) is spread over enough rows: staged for rows of
//     at least 12 units (24 and more: 8 waves, 4 in flight, split staging,
//     two rows per wave where that pads less), for rows of 4-11 units with
//     more than 16 rows per CU (4 waves, split staging, at most 2
//     workgroups per CU), or for 8192 rows and more; read with each unit
//     otherwise (two rows per wave from 5 units).  Rows
//     whose staged x passes 64 KiB stage it up to the device's LDS per
//     workgroup (8 waves, 4 in flight, x before A, one workgroup per CU),
//     reading x with each unit beyond that.
// Two rows per wave are taken only where the halved grid still gives every
// CU a workgroup.  With a cap the grid stays below the row count and waves
// walk several rows; otherwise every launch gives each CU work once
// M >= CUs.
Plan rows_plan(int kind, int M, int N, bool aligned, const Device& dev)
{
    Plan p{};
    const int cus = dev.cus;
    const int epc = elems_per_chunk(kind);
    // The streaming kernel addresses a row through a 32-bit byte count (the
    // INT8/INT4 buffer resource's range, the row stride): rows of 2 GiB or
    // more take the element-wise kernel, which uses 64-bit offsets.  Its row
    // cursors (and the packed kernel's group cursors) run up to about twice
    // M in int: more than 2^30 rows also take the element-wise kernel.
    const bool huge_row = (int64_t)(N / epc) * 16 >= ((int64_t)1 << 31);
    const bool huge_m = M > (1 << 30);
    if (!aligned || N == 0 || N % epc != 0 || huge_row || huge_m) {
        p.variant = 3;
        p.block = 256;
        p.waves = 4;
        p.grid = gemv_device::capped_grid(((int64_t)M + 3) / 4, p.block);
        p.rows = 1;
        p.D = 1;
        return p;
    }
    const int nchunks = N / epc;
    const int P = (nchunks + 63) / 64;
    // row groups of a packed launch (rows of at most 32 chunks only)
    const int64_t packed_groups = nchunks <= kPackedMaxChunks
                                      ? ((int64_t)M + packed_rows_per_load(nchunks) - 1) / packed_rows_per_load(nchunks)
                                      : 0;
    if ((kind == kQ8 || kind == kQ4) && nchunks <= kPackedMaxChunks && packed_groups > 3 * (int64_t)cus) {
        // more than 3 row groups per CU (fewer: x in registers, a wave per
        // row, was 5-18 % faster on 12 such shapes)
        const int64_t groups = packed_groups;
        const int64_t per_cu = (groups + cus - 1) / cus;
        p.variant = 4;
        p.waves = 8;
        // one group per wave up to 16 per CU, two (both in flight) up to 80,
        // beyond that four, two rounds of two (four groups per wave lost
        // below 80 per CU: INT4 40979 x 512 5.73 -> 4.79 us, INT8 30962 x
        // 384 4.87 -> 4.67; won above: INT4 61267 x 896 9.28 -> 8.32)
        p.D = per_cu <= 16 ? 1 : 2;
        p.rows = per_cu <= 80 ? p.D : 4;
        p.stg = -1;   // x goes straight to registers
        p.lds = 0;
        p.block = p.waves * 64;
        const int64_t waves_needed = (groups + p.rows - 1) / p.rows;
        p.grid = gemv_device::capped_grid((waves_needed + p.waves - 1) / p.waves, p.block);
        return p;
    }
    const bool fp = kind == kF32 || kind == kF16 || kind == kF16H;
    if (P == 1 && (!fp || M <= 32 * cus)) {
        // rows of one unit: x in registers
        p.variant = 5;
        p.xk = 1;
        p.rows = 1;
        if (M <= 32 * cus) {
            p.waves = fp ? 8 : 4;
            p.D = 1;
        } else if (M <= 64 * cus) {
            p.waves = 4;
            p.D = 2;
            p.rows = 2;
        } else {
            p.waves = 8;
            p.D = 2;
            p.cap = 3;
        }
    } else if (P == 2 && (fp || (kind == kQ4 && M <= 16 * cus) || (kind == kF16X32 && M > 16 * cus))) {
        // rows of two units: x in registers
        p.variant = 5;
        p.xk = 2;
        p.rows = 1;
        p.waves = 4;
        p.D = 2;
        p.cap = kind == kF16X32 ? 6 : 0;
    } else if (P == 3 && (fp || kind == kF16X32 || (kind == kQ4 && M <= 8 * cus))) {
        // rows of three units: x in registers
        p.variant = 5;
        p.xk = 3;
        p.rows = 1;
        p.D = 3;
        if (fp) {
            p.waves = M <= 32 * cus ? 8 : 4;
        } else if (kind == kF16X32 && M > 16 * cus) {
            p.waves = 8;
            p.cap = 3;
        } else {
            // 4 waves: with 8, few INT4 rows left most CUs idle (328 x 5248
            // 3.42 -> 2.81 us)
            p.waves = 4;
        }
    } else if (fp) {
        p.variant = 2;
        if (P >= 24) {
            // very long rows: 4 waves; up to 11 rows per CU two rows per
            // wave, 8 in flight (few enough waves that split_plan takes
            // over: two waves per row); from 11 to 16 rows per CU four rows
            // per wave, 8 in flight, so that the grid gives every CU one
            // workgroup (four_rows_rule), except rows of a multiple of 16
            // units (FP16 4096 x 32768 42.31 us against 43.18 with four);
            // from 24 rows per CU 8 in flight, one row per wave (two where a
            // row's units are not a multiple of 8, which would pad every
            // row's stream); in between two rows per wave, 4 in flight
            p.waves = 4;
            if (M <= 11 * cus) {
                p.D = 8;
                p.rows = 2;
            } else if (M <= 16 * cus && P % 16 != 0) {
                p.D = 8;
                p.rows = 4;
            } else if (M >= 24 * cus || P % 16 == 0) {
                // (between 12 and 24 rows per CU only rows of a multiple of
                // 16 units measured faster so: FP16 4096 x 32768 44.5 ->
                // 42.3 us, 4096 x 16384 22.1 -> 21.4)
                p.D = 8;
                p.rows = P % 8 == 0 ? 1 : 2;
            } else {
                p.D = 4;
                p.rows = 2;
            }
        } else if (P >= 4) {
            p.waves = P >= 16 ? 8 : 4;
            least_padding(P, two_rows_fill(M, p.waves, cus), &p.D, &p.rows);
        } else {
            // rows of 1-3 units: enough rows per wave for 4 units in flight
            // (one row per wave would pad each wave's stream with re-reads)
            p.waves = P == 1 ? 8 : 4;
            p.D = 4;
            p.rows = (4 + P - 1) / P;
        }
    } else if (kind == kF16X32) {
        // (up to 7 rows per CU of 4 units and more: split rows, split_plan)
        const int64_t lds = lds_bytes(kind, nchunks);
        const bool fits = lds <= dev.lds_max;
        p.rows = 1;
        if (fits && P >= 12 && M > 8 * cus && M <= 14 * cus) {
            // rows of 12 units and more, 8-14 rows per CU: 8 waves, 4 in
            // flight, two rows per wave (fewer stagings of x), split staging,
            // no cap.  Brute force over every plan on 7 such shapes (8-13
            // rows per CU): at most 3.4 % from the fastest, against 2.6-19.5 %
            // (2111 x 8704 11.21 -> 9.38 us, 3046 x 12672 15.93 -> 14.09)
            p.variant = 1;
            p.waves = 8;
            p.D = 4;
            p.stg = 2;
            p.rows = 2;
        } else if (fits && P == 16) {
            // rows of 16 units: 8 waves, 8 in flight, A first, at most 3
            // workgroups per CU (8192 x 8192 22.45 us, against 22.66 for
            // the rule below)
            p.variant = 1;
            p.waves = 8;
            p.D = 8;
            p.stg = 0;
            p.cap = 3;
        } else if (fits && P >= 4) {
            // staged x, 4 waves, split staging; rows of 11 units and more 8
            // in flight, shorter ones 4; at most 2 workgroups per CU, one
            // for rows of 16 units and more.  Brute force over every plan
            // on 120 seeded random shapes (these rules and the split rows
            // together): 2.3 % from the fastest (geometric mean; 9.5 % at
            // worst), against 4.1 % (31 %) for the rules before, which took
            // 8 waves for rows of 12 units and more (12815 x 14720 63.57 ->
            // 57.20 us, 4137 x 19968 32.51 -> 30.01)
            p.variant = 1;
            p.waves = 4;
            p.stg = 2;
            p.D = P >= 11 ? 8 : 4;
            p.cap = P >= 16 ? 1 : 2;
        } else if (fits && M >= 8192) {
            p.variant = 1;
            p.waves = 4;
            p.D = 8;
            p.cap = 4;
        } else {
            p.variant = 2;
            // 4 waves; rows of 8 units or more: two per wave, 8 in flight;
            // 4 units: one row, 4 in flight; 5-7 units: two rows (less
            // padding: 2048 x 3072 4.37 -> 4.21 us); shorter: 4 units in
            // flight over ceil(4 / P) rows
            p.waves = 4;
            p.D = P >= 8 ? 8 : 4;
            p.rows = P >= 8 ? 2 : (P == 4 ? 1 : (P > 4 ? (two_rows_fill(M, 4, cus) ? 2 : 1) : (4 + P - 1) / P));
        }
    } else if (kind == kQ8) {
        p.variant = 1;
        p.D = 4;
        p.rows = 1;
        const int64_t lds = lds_bytes(kind, nchunks);
        if (lds > dev.lds_max || (lds >= kLdsBytes && 2 * lds > dev.lds_max && M <= 8 * cus)) {
            // staged x would not fit a workgroup, or only one workgroup
            // per CU and few rows to spread its staging over: x read with
            // each unit, 4 waves of two rows each, 8 units in flight
            p.variant = 2;
            p.waves = 4;
            p.D = 8;
            p.rows = 2;
        } else if (lds >= kLdsBytes) {
            // long rows (32 units and more), staged x of 64 KiB or more: 4 waves, split
            // staging, at most 2 workgroups per CU when two fit and the
            // rows are many; else 8 waves, x staged before A, one
            // workgroup per CU
            const bool two = 2 * (lds + kSplitSpareBytes) <= dev.lds_max && M > 4 * cus;
            p.waves = two ? 4 : 8;
            p.stg = two ? 2 : 1;
            p.cap = two ? 2 : 1;
        } else if (P == 2 && M <= 16 * cus) {
            // few rows of two units: x read with each unit (no staging, no
            // barrier), 4 waves, 2 in flight (8 waves: 1.7 % slower on 7
            // shapes, 2115 x 2048 3.24 -> 3.09 us)
            p.variant = 2;
            p.waves = 4;
            p.D = 2;
        } else if (P >= 8 && M <= 4 * cus) {
            // rows of 8-32 units, at most 4 per CU: 8 waves, x staged before
            // A, one workgroup per CU
            p.waves = 8;
            p.stg = 1;
            p.cap = 1;
        } else if (P <= 16 && M <= 8 * cus) {
            // few rows (one GPU's share of a row-split matrix): x read with
            // each unit, 4 in flight; 8 waves, 4 below 4 rows per CU (so
            // that every CU gets a workgroup: 736 x 2560 2.97 -> 2.54 us)
            p.variant = 2;
            p.waves = M < 4 * cus ? 4 : 8;
        } else if (P >= 8) {
            // rows of 8-31 units, many of them: 4 waves, split staging; rows
            // of 8-10 units two per wave with no cap where that still gives
            // every CU a workgroup (8192 x 8192 12.11 -> 11.66 us), longer
            // ones one per wave, at most 2 workgroups per CU.  Brute force
            // over every plan on 27 such shapes: 3.8 % from the fastest
            // (geometric mean), against 8.2 % for the earlier rule (8 waves,
            // A first; 12 waves at 20-32 rows per CU), which the exact INT8
            // decode left behind (6618 x 15104 20.37 -> 18.69 us)
            p.waves = 4;
            p.stg = 2;
            if (P <= 10 && two_rows_fill(M, 4, cus)) {
                p.rows = 2;
            } else {
                p.cap = 2;
            }
        } else if (P <= 2) {
            // rows of 2 units: 8 waves, 2 in flight, split staging, at most
            // 3 workgroups per CU (waves walk several rows)
            p.waves = 8;
            p.D = 2;
            p.stg = 2;
            p.cap = 3;
        } else {
            // rows of 3-7 units, many of them: 4 waves, split staging, at
            // most 3 workgroups per CU for rows of 3-5 units, 5 in flight for
            // rows of 5 (no padding: 14336 x 5120 13.28 -> 12.86 us; rows of
            // 3: 10225 x 2304 7.35 -> 6.21, 3564 x 2064 4.81 -> 3.72); rows of
            // 6 and 7 units at most 4 (against 8 waves, A first, at most 2:
            // 4525 x 6912 8.94 -> 7.15 us, 5744 x 6400 9.35 -> 8.28)
            p.waves = 4;
            p.stg = 2;
            p.cap = P <= 5 ? 3 : 4;
            p.D = P == 5 ? 5 : 4;
        }
    } else if (const int64_t lds = lds_bytes(kind, nchunks); lds > dev.lds_max || M <= 4 * cus) {
        // INT4 rows whose staged x would not fit a workgroup, or at most 4
        // rows per CU (of 4 units or more: shorter ones took x in
        // registers): x read with each unit, 4 waves, 4 in flight
        p.variant = 2;
        p.waves = 4;
        p.D = 4;
        p.rows = 1;
    } else if (lds > kLdsBytes) {
        // long INT4 rows, staged x past 64 KiB: 8 waves, 4 in
        // flight, x staged before A, one workgroup per CU
        p.variant = 1;
        p.waves = 8;
        p.D = 4;
        p.rows = 1;
        p.stg = 1;
        p.cap = 1;
    } else {
        // short INT4 rows: 8 waves, 2 units in flight, split staging, at
        // most 4 workgroups per CU (3 measured 1.7-4.8 % slower on seven
        // shapes: 14336 x 4096 7.52 -> 7.30 us); rows of 5-9 units: 4
        // units in flight (5 and 3 for rows of 5 and 6 units, which divide
        // them: 2048 x 10240 5.65 -> 5.08 us, 2048 x 12288 5.65 -> 5.42), x
        // staged before A, 4 waves and at most 3 workgroups per CU.  With x
        // in per-pass planes (staged_index), brute force over every plan on
        // 72 seeded random shapes moved rows of 10 units and more, and many
        // rows of 4, to 8 waves, 4 in flight, split staging and 1 (2 for
        // rows of 4) workgroups per CU: the picks from 1.9 % to 1.0 % behind
        // the fastest plan (geometric mean; 12.2 % to 6.8 % at worst;
        // 5832 x 25088 17.2 -> 15.4 us, 4096 x 8192 5.77 -> 5.49)
        p.variant = 1;
        p.rows = 1;
        if (P >= 10 || (P == 4 && M > 8 * cus)) {
            p.waves = 8;
            p.D = 4;
            p.stg = 2;
            p.cap = P >= 10 ? 1 : 2;
        } else {
            p.waves = P < 4 ? 8 : 4;
            p.D = P < 4 ? 2 : (P == 5 ? 5 : (P == 6 ? 3 : 4));
            p.stg = P < 4 ? 2 : 1;
            p.cap = P < 4 ? 4 : 3;
        }
    }
    // staged plans were chosen only where x fits the device's LDS
    p.lds = p.variant == 1 ? (int)lds_bytes(kind, nchunks) : 0;
    if (p.variant == 1 && p.stg == 2) {
        // split staging writes past-the-end granules to spare slots
        if (p.lds + kSplitSpareBytes <= dev.lds_max)
            p.lds += kSplitSpareBytes;
        else
            p.stg = 1;
    }
    finish_rows(M, cus, &p);
    return p;
}

// FP32/FP16 cost model: the predicted time of a plan from its geometry.  A
// launch has a fixed cost (the same for every plan; it matters only to the
// margin below, which is relative).  A wave streams
// U units -- its rows' units padded to a multiple of D -- D at a time, so
// it waits about U/D + 1 memory latencies; the busiest CU runs
// ceil(grid / CUs) workgroups, in turn where they outnumber the workgroups
// it holds at once (its 4 SIMDs hold waves-per-SIMD x 4 waves, so that
// many / waves workgroups); the chip streams every unit at the HBM rate, a
// walking wave's padding included (it re-reads its last row from the
// start), a split row's not (its padded loads repeat the wave's own last
// unit, served from the caches); a CU streams its units at a per-CU rate
// and issues a fixed cost per unit on its 4 SIMDs.
// The four times overlap only in part and combine as a root sum of squares;
// split rows add their LDS reduction.  The constants were fitted (weighted
// least squares on log time, near-best plans weighted most) to the
// graph-timed times of every candidate plan below on 52 seeded random
// FP32/FP16 shapes on MI355X; they read as a launch cost of 1.69 us, a
// latency of 0.34 us per round,
// 8.9 TB/s for the chip, 47 GB/s per CU and 18 / 26 ns of issue per unit
// and wave for FP32 / FP16.  On 32 further random shapes the plan the model
// picks (within the margin below) is 3.4 % slower than the fastest
// candidate (geometric mean; 10.5 % at worst for FP16, 17 % for FP32),
// the measured rules alone 6.3 % (34 % at worst).  The two corrections
// above (the fit predates them: it held 8 two-wave workgroups per CU, and
// counted split rows' padding as traffic) take the picks on 144 random
// shapes from 4.3 % to 3.9 % (FP32) and 3.9 % to 3.4 % (FP16) behind the
// fastest plan (FP16 799 x 9344 5.87 -> 4.93 us, 10463 x 3200 13.75 ->
// 11.65: two waves per row); refitting the constants in the corrected
// form made held-out picks worse in five of six folds, so they stay.
struct FpCostModel {
    double launch;        // s, fixed cost of a launch
    double latency;       // s per memory round trip under load
    double chip_bw;       // B/s, all CUs
    double cu_bw;         // B/s, one CU
    double split_cost;    // s, LDS reduction of a split row
    double issue[2];      // s per unit and wave: FP32, FP16
};
constexpr FpCostModel kFpModel{1.691e-6, 3.412e-7, 8.946e12, 4.670e10, 1.814e-8, {1.788e-8, 2.597e-8}};

// The model replaces the measured rules' plan only where it predicts a gain
// above its own error on the rules' home ground: on the shapes the rules
// were tuned on it ranks plans within 3-5 % of each other wrongly about as
// often as rightly.
constexpr double kModelMargin = 1.05;

// The fitted shapes' range (row counts and lengths drawn log-uniform from
// these): outside it the measured rules alone decide.
constexpr int kModelRows[2] = {256, 65536};
constexpr int kModelCols[2] = {256, 32768};

// Waves one SIMD holds: the FP32/FP16 streaming kernels with 8 units in
// flight use 68-69 VGPRs (7 waves of 512 registers); every other FP32/FP16
// kernel uses at most 39 (8 waves, the hardware's limit).
int fp_waves_per_simd(const Plan& p) { return p.variant == 2 && p.D == 8 ? 7 : 8; }

double fp_cost(int kind, int64_t M, int64_t P, int cus, const Plan& p)
{
    const FpCostModel& m = kFpModel;
    const int64_t waves = (int64_t)p.grid * p.waves;
    int64_t U = 0, units = 0;
    if (p.variant == 6) {
        U = ((P + p.xk - 1) / p.xk + p.D - 1) / p.D * p.D;
        units = M * P;   // padding re-reads the wave's last unit from cache
    } else {
        // waves 0 .. nmax-1 walk rmax rows, the others rmin
        const int64_t PP = p.variant == 5 ? p.xk : P;
        const int64_t rmax = (M + waves - 1) / waves, rmin = M / waves, nmax = M - rmin * waves;
        U = (rmax * PP + p.D - 1) / p.D * p.D;
        const int64_t Umin = (rmin * PP + p.D - 1) / p.D * p.D;
        units = nmax * U + (waves - nmax) * Umin;
    }
    const int held = std::min(4 * fp_waves_per_simd(p) / p.waves, 32);   // workgroups per CU
    const int64_t wgs = (p.grid + cus - 1) / cus;                                 // on the busiest CU
    const double rounds = std::max((double)wgs / held, 1.0) * ((double)U / p.D + 1.0);
    const double cu_units = (double)wgs * p.waves * U;
    const double t_chip = (double)units * 1024.0 / m.chip_bw;
    const double t_cu = cu_units * 1024.0 / m.cu_bw;
    const double t_lat = rounds * m.latency;
    const double t_issue = cu_units * m.issue[kind == kF16 ? 1 : 0] / 4.0;
    return m.launch + (p.variant == 6 ? m.split_cost : 0.0) +
           std::sqrt(t_chip * t_chip + t_cu * t_cu + t_lat * t_lat + t_issue * t_issue);
}

// FP32/FP16: the measured rules' plan p0, or the candidate the cost model
// ranks fastest where it predicts more than kModelMargin of a gain.
// Candidates: the streaming kernel with 4 or 8 waves, 2, 4 or 8 units in
// flight and 1, 2 or 4 rows per wave; rows of 1-3 units with x in
// registers; split rows of S = 2-16 waves (each at least two units) with 2
// or 4 in flight.
Plan fp_model_plan(int kind, int M, int P, const Device& dev, const Plan& p0)
{
    double best_t = fp_cost(kind, M, P, dev.cus, p0);
    const double rules_t = best_t;
    Plan best = p0;
    auto consider = [&](const Plan& c) {
        const double t = fp_cost(kind, M, P, dev.cus, c);
        if (t < best_t) {
            best_t = t;
            best = c;
        }
    };
    auto rows_candidate = [&](int variant, int waves, int D, int rows, int cap, int xk) {
        Plan c{};
        c.variant = variant;
        c.waves = waves;
        c.D = D;
        c.rows = rows;
        c.cap = cap;
        c.xk = xk;
        c.stg = -1;
        finish_rows(M, dev.cus, &c);
        consider(c);
    };
    if (P == 1) {
        for (int waves : {4, 8})
            for (int D : {1, 2})
                for (int rows : {1, 2})
                    for (int cap : {0, 3})
                        rows_candidate(5, waves, D, rows, cap, 1);
    } else if (P == 2) {
        for (int cap : {0, 3, 6})
            rows_candidate(5, 4, 2, 1, cap, 2);
    } else if (P == 3) {
        for (int waves : {4, 8})
            for (int cap : {0, 3})
                rows_candidate(5, waves, 3, 1, cap, 3);
    }
    for (int waves : {4, 8})
        for (int D : {2, 4, 8})
            for (int rows : {1, 2, 4})
                rows_candidate(2, waves, D, rows, 0, 0);
    for (int S : {2, 4, 8, 16}) {
        // one workgroup per row, no walking: the grid must hold every row
        if (2 * S > P || (int64_t)M * S * 64 > gemv_device::kMaxWorkItems)
            continue;
        // from two rows per CU split rows keep the rules' two waves per row:
        // on three seeds of random shapes the model's 4-16 waves per row
        // there lost to two in 9 of 11 shapes (FP32 1399 x 28288 29.53 ->
        // 26.76 us, 581 x 23168 12.95 -> 11.58, FP16 1071 x 29440 13.84 ->
        // 12.65; the two it won by 0.8-1.6 %)
        if (S > 2 && M >= 2 * (int64_t)dev.cus)
            continue;
        for (int D : {2, 4}) {
            Plan c{};
            c.variant = 6;
            c.xk = S;
            c.waves = S;
            c.block = S * 64;
            c.D = D;
            c.rows = 1;
            c.stg = -1;
            c.grid = M;
            consider(c);
        }
    }
    return rules_t > kModelMargin * best_t ? best : p0;
}

// FP32/FP16 rows of 24 units and more, 11-16 rows per CU: 4 waves of four
// rows each, 8 in flight, one workgroup per CU (rows_plan), a measured rule
// that neither split_plan nor the cost model replaces.  Brute force over
// every plan on 16 seeded random shapes there: the fastest plan on 13 (9 %
// behind at worst, 2856 x 28928 at 11.2 rows per CU), where the split rows
// and the cost model's picks were 0-15 % behind (FP32 3912 x 6784 19.52 ->
// 16.97 us, 3494 x 10880 27.41 -> 24.45, FP16 3656 x 26752 33.70 -> 30.18);
// past 16 rows per CU some CUs get two workgroups and it falls 37-58 %
// behind.
bool four_rows_rule(const Plan& p) { return (p.variant == 2 && p.rows == 4 && p.waves == 4 && p.D == 8); }

// Row slabs (variant 7, gemv_slab) for INT8, INT4 and FP16 with FP32 x,
// whose x the streaming kernel stages in LDS once per workgroup or reads
// with every unit.  A slab plan takes S = P waves per workgroup (S = P / 2,
// two passes per wave, for rows of 17-32 units and INT8 rows of an even
// count from 10), 4 rows per slab, 4 loads in flight (8 with two passes
// per wave).  Where it is taken: FP16 with FP32 x from one row per CU, for
// rows of 2 units and more, and one-unit rows from 14 rows per CU; INT4
// rows of 3-16 units but 6, from one row per CU (rows of 8 units and more
// only up to 12 rows per CU), and one-unit rows of more than 32 chunks
// (past the packed kernel) from 4 rows per CU; INT8 rows of 9 units and
// more between 2 and 12 rows per CU.  Slabs of 8 rows where two passes
// per wave give the busiest CU no more rows than slabs of 4 (fewer
// workgroups, each loading its x once) and every CU still a slab.  INT4 caps the grid at 32 waves per
// CU, so that workgroups walk several slabs with x loaded once.
// Graph-timed on four seeds of 24 random shapes per format (bench-style
// ring over >= 1 GiB), against the rules before: geometric mean 0.957 /
// 0.945 (FP16 with FP32 x, seeds 0-1 / 2-3), 0.968 / 0.964 (INT4), 0.990 /
// 0.988 (INT8), with no INT shape slower by more than 3 %: INT4 4096 x
// 14336 8.08 -> 7.84 us, FP16 with FP32 x 8192 x 8192 22.82 -> 22.02,
// INT8 2295 x 24576 14.51 -> 12.21, INT4 569 x 8320 4.16 -> 3.25.  Rows of
// 2 units (INT4 14336 x 4096 7.30 -> 7.74), INT8 rows of 4-8 units (14336 x
// 4096 10.74 -> 11.15, 8192 x 8192 12.39 -> 12.74) and INT4 rows of 6
// units (5113 x 10880 8.17 -> 8.79) stay with the streaming kernel.  A
// fifth seed, held out (the plan search, every candidate timed): INT4 0.937
// and FP16 with FP32 x 0.962 of the previous planner's times, INT8 1.001;
// its INT4 one-unit rows past the packed kernel (51636 x 1408 10.34 ->
// 9.18 us, 26708 x 1536 7.20 -> 6.53) and INT8 rows of 16 units (4039 x
// 15616 12.47 at one pass per wave, 11.57-11.86 at two) gave the last two
// rules, which the four training seeds support too (INT4 22965 x 2048
// 7.27 -> 6.73; INT8 2567 x 15616 10.71 -> 9.04 at two passes, 9.16 at
// one).  A sixth seed, held out after that: row slabs 0.913 (INT4, 6
// shapes) and 0.974 (FP16 with FP32 x, 18 shapes) of the fastest plan of
// the other kernels, but INT8 1.070 (7 shapes), its losses all past 12 rows
// per CU (5559 x 13312 16.69 against 13.78, 12805 x 12672 31.52 against
// 26.20, 4008 x 18432 14.33 against 13.52): INT8 row slabs stop at 12 rows
// per CU (all six seeds: 0.988-1.003 of the streaming kernels' best over
// every INT8 shape, where up to 100 rows per CU read 0.986-1.018).
bool slab_plan(int kind, int M, int nchunks, int cus, Plan* p)
{
    const int P = (nchunks + 63) / 64;
    const int64_t rows = M;
    bool take = false;
    if (kind == kF16X32)
        take = rows >= cus && (P >= 2 || rows >= 14 * (int64_t)cus);
    else if (kind == kQ4)
        take = (rows >= cus && P >= 3 && P <= 16 && P != 6 && (P <= 7 || rows <= 12 * (int64_t)cus)) ||
               (P == 1 && nchunks > kPackedMaxChunks && rows >= 4 * (int64_t)cus);
    else if (kind == kQ8)
        take = P >= 9 && rows >= 2 * (int64_t)cus && rows <= 12 * (int64_t)cus;
    if (!take || P > 32 || (P > 16 && P % 2 != 0))
        return false;
    // two passes per wave for rows of 17-32 units, and for INT8 rows of an
    // even count from 10 units
    const int S = P > 16 || (kind == kQ8 && P >= 10 && P % 2 == 0) ? P / 2 : P;
    const int Q = P / S;
    int R = 4;
    if (Q == 2) {
        // rows on the busiest CU: whole slabs, grid of one slab per workgroup
        auto busiest = [&](int r) { return ((rows + r - 1) / r + cus - 1) / cus * r; };
        if ((rows + 7) / 8 >= cus && busiest(8) <= busiest(4))
            R = 8;
    }
    *p = Plan{};
    p->variant = 7;
    p->waves = S;
    p->block = S * 64;
    p->xk = Q;
    p->rows = R;
    p->D = Q == 2 ? 8 : 4;
    p->stg = -1;
    p->lds = 0;
    int64_t grid = (rows + R - 1) / R;
    if (kind == kQ4) {
        const int64_t cap = (int64_t)(32 / S > 1 ? 32 / S : 1) * cus;
        if (grid > cap) {
            grid = cap;
            p->cap = 32 / S > 1 ? 32 / S : 1;
        }
    }
    p->grid = gemv_device::capped_grid(grid, p->block);
    return true;
}

Plan plan_uncached(int kind, int M, int N, bool aligned, const Device& dev)
{
    const Plan p0 = rows_plan(kind, M, N, aligned, dev);
    if (p0.variant == 3 || ((kind == kF32 || kind == kF16) && four_rows_rule(p0)))
        return p0;
    const int P = (N / elems_per_chunk(kind) + 63) / 64;
    Plan sl{};
    if (slab_plan(kind, M, N / elems_per_chunk(kind), dev.cus, &sl))
        return sl;
    Plan p = p0;
    Plan s{};
    if (split_plan(kind, M, P, dev.cus, p0, &s))
        p = s;
    // the model only within the shapes it was fitted on
    const bool fitted = M >= kModelRows[0] && M <= kModelRows[1] && N >= kModelCols[0] && N <= kModelCols[1];
    return (kind == kF32 || kind == kF16) && fitted ? fp_model_plan(kind, M, P, dev, p) : p;
}

// The plan of a call: the one-wave-per-row plan (rows_plan), or split rows
// where that leaves the CUs short of waves; for FP32/FP16 then the cost
// model's choice where it predicts a clear gain.  Each host thread keeps
// its last 16 plans, so repeated calls of a shape skip the search.
Plan make_plan(int kind, int M, int N, bool aligned, const Device& dev)
{
    struct Entry {
        int kind, M, N, cus, lds_max;
        bool aligned, used;
        Plan p;
    };
    constexpr int kEntries = 16;
    static thread_local Entry cache[kEntries];
    static thread_local unsigned next = 0;
    for (const Entry& e : cache)
        if (e.used && e.kind == kind && e.M == M && e.N == N && e.aligned == aligned && e.cus == dev.cus &&
            e.lds_max == dev.lds_max)
            return e.p;
    const Plan p = plan_uncached(kind, M, N, aligned, dev);
    cache[next++ % kEntries] = Entry{kind, M, N, dev.cus, dev.lds_max, aligned, true, p};
    return p;
}

template <int F>
const void* select_packed(const Plan& p)
{
    return p.D == 1 ? reinterpret_cast<const void*>(&gemv_packed<F, 8, 1>)
                    : reinterpret_cast<const void*>(&gemv_packed<F, 8, 2>);
}

template <int F, int S>
const void* select_split_d(const Plan& p)
{
    return p.D == 2 ? reinterpret_cast<const void*>(&gemv_split<F, S, 2>)
                    : reinterpret_cast<const void*>(&gemv_split<F, S, 4>);
}

template <int F>
const void* select_split(const Plan& p)
{
    switch (p.xk) {
    case 2: return select_split_d<F, 2>(p);
    case 4: return select_split_d<F, 4>(p);
    case 8: return select_split_d<F, 8>(p);
    default: return select_split_d<F, 16>(p);
    }
}

template <int F, int Q, int R>
const void* select_slab_r(const Plan& p)
{
    if constexpr (R * Q >= 8) {
        if (p.D == 8)
            return reinterpret_cast<const void*>(&gemv_slab<F, Q, 8, R>);
    }
    return reinterpret_cast<const void*>(&gemv_slab<F, Q, 4, R>);
}

template <int F, int Q>
const void* select_slab_q(const Plan& p)
{
    return p.rows == 4 ? select_slab_r<F, Q, 4>(p) : select_slab_r<F, Q, 8>(p);
}

template <int F>
const void* select_slab(const Plan& p)
{
    return p.xk == 2 ? select_slab_q<F, 2>(p) : select_slab_q<F, 1>(p);
}

template <int F>
const void* select_xreg(const Plan& p)
{
    if (p.xk == 3)
        return p.waves == 8 ? reinterpret_cast<const void*>(&gemv_xreg<F, 8, 3, 3>)
                            : reinterpret_cast<const void*>(&gemv_xreg<F, 4, 3, 3>);
    if (p.xk == 2)
        return reinterpret_cast<const void*>(&gemv_xreg<F, 4, 2, 2>);
    if (p.D == 2)
        return p.waves == 8 ? reinterpret_cast<const void*>(&gemv_xreg<F, 8, 2, 1>)
                            : reinterpret_cast<const void*>(&gemv_xreg<F, 4, 2, 1>);
    return p.waves == 8 ? reinterpret_cast<const void*>(&gemv_xreg<F, 8, 1, 1>)
                        : reinterpret_cast<const void*>(&gemv_xreg<F, 4, 1, 1>);
}

template <int F, int W, int D, bool XG, int STG>
const void* stream_kernel()
{
    return reinterpret_cast<const void*>(&gemv_stream<F, W, D, kNT, XG, STG>);
}

template <int F, bool XG, int STG>
const void* select_stream_stg(const Plan& p)
{
    // in-flight depths that divide rows of 5 or 6 units (4 waves)
    if constexpr ((F == kQ8 && !XG && STG == 2) || (F == kQ4 && !XG && STG == 1)) {
        if (p.waves == 4 && p.D == 5)
            return stream_kernel<F, 4, 5, XG, STG>();
    }
    if constexpr (F == kQ4 && !XG && STG == 1) {
        if (p.waves == 4 && p.D == 3)
            return stream_kernel<F, 4, 3, XG, STG>();
    }
    if (p.waves == 8)
        return p.D == 8 ? stream_kernel<F, 8, 8, XG, STG>()
                        : (p.D == 4 ? stream_kernel<F, 8, 4, XG, STG>() : stream_kernel<F, 8, 2, XG, STG>());
    return p.D == 8 ? stream_kernel<F, 4, 8, XG, STG>()
                    : (p.D == 4 ? stream_kernel<F, 4, 4, XG, STG>() : stream_kernel<F, 4, 2, XG, STG>());
}

template <int F, bool XG>
const void* select_stream(const Plan& p)
{
    if constexpr (XG)
        return select_stream_stg<F, XG, 0>(p);   // nothing is staged
    else
        return p.stg == 2 ? select_stream_stg<F, XG, 2>(p)
                          : (p.stg == 1 ? select_stream_stg<F, XG, 1>(p) : select_stream_stg<F, XG, 0>(p));
}

// Variant 1 stages x in LDS, variant 2 reads it with each unit; FP32 and
// FP16 always take variant 2.
template <int F>
const void* select_kernel(const Plan& p)
{
    if (p.variant == 3)
        return reinterpret_cast<const void*>(&gemv_elementwise<F>);
    if (p.variant == 5)
        return select_xreg<F>(p);
    if constexpr (F != kF16H) {
        if (p.variant == 6)
            return select_split<F>(p);
    }
    if constexpr (F == kQ8 || F == kQ4) {
        if (p.variant == 4)
            return select_packed<F>(p);
    }
    if constexpr (F == kQ8 || F == kQ4 || F == kF16X32) {
        if (p.variant == 7)
            return select_slab<F>(p);
    }
    if constexpr (F == kF32 || F == kF16 || F == kF16H)
        return select_stream<F, true>(p);
    else
        return p.variant == 2 ? select_stream<F, true>(p) : select_stream<F, false>(p);
}

const void* kernel_for(int kind, const Plan& p)
{
    switch (kind) {
    case kF32: return select_kernel<kF32>(p);
    case kF16: return select_kernel<kF16>(p);
    case kQ8: return select_kernel<kQ8>(p);
    case kF16X32: return select_kernel<kF16X32>(p);
    case kF16H: return select_kernel<kF16H>(p);
    default: return select_kernel<kQ4>(p);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Enqueue plan p on `stream`.
int launch_planned(int kind, const Plan& p, const void* A, const uint16_t* scale, const void* x, float* y, int M,
                   int N, hipStream_t stream)
{
    const uint8_t* a8 = static_cast<const uint8_t*>(A);
    const uint8_t* x8 = static_cast<const uint8_t*>(x);
    void* args[] = {(void*)&a8, (void*)&scale, (void*)&x8, (void*)&y, (void*)&M, (void*)&N};
    const hipError_t err = hipLaunchKernel(kernel_for(kind, p), dim3(p.grid), dim3(p.block), args,
                                           (size_t)p.lds, stream);
    return err == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}

int launch(int kind, const void* A, const uint16_t* scale, const void* x, float* y, int M, int N,
           hipStream_t stream)
{
    if (M < 0 || N < 0)
        return GEMV_E_INVAL;
    if (kind == kQ4 && N % 128 != 0)
        return GEMV_E_UNSUPPORTED;
    if (M == 0)
        return GEMV_OK;
    if (y == nullptr)
        return GEMV_E_INVAL;
    if (N > 0 && (A == nullptr || x == nullptr))
        return GEMV_E_INVAL;
    if ((kind == kQ8 || kind == kQ4) && N > 0 && scale == nullptr)
        return GEMV_E_INVAL;
    Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    const bool aligned = aligned16(A) && aligned16(x);
    const Plan p = make_plan(kind, M, N, aligned, dev);
    return launch_planned(kind, p, A, scale, x, y, M, N, stream);
}

// Probe geometry: enough 256-thread workgroups to give every CU 8 of them.
constexpr int kProbeU = 4;
constexpr int kProbeWgPerCu = 8;

int probe_grid(int64_t n16, int* grid)
{
    Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    const int cus = dev.cus;
    const int64_t per_wg = 256 * kProbeU;
    const int64_t need = (n16 + per_wg - 1) / per_wg;
    const int64_t cap = (int64_t)cus * kProbeWgPerCu;
    *grid = (int)(need < cap ? need : cap);
    return GEMV_OK;
}

}  // namespace
}  // namespace gemv

extern "C" {

int gemv_f32(const float* A, const float* x, float* y, int M, int N, hipStream_t stream)
{
    return gemv::launch(gemv::kF32, A, nullptr, x, y, M, N, stream);
}

int gemv_f16(const uint16_t* A, const uint16_t* x, float* y, int M, int N, hipStream_t stream)
{
    return gemv::launch(gemv::kF16, A, nullptr, x, y, M, N, stream);
}

int gemv_f16x32(const uint16_t* A, const float* x, float* y, int M, int N, hipStream_t stream)
{
    return gemv::launch(gemv::kF16X32, A, nullptr, x, y, M, N, stream);
}

int gemv_f16_acc16(const uint16_t* A, const uint16_t* x, float* y, int M, int N, hipStream_t stream)
{
    return gemv::launch(gemv::kF16H, A, nullptr, x, y, M, N, stream);
}

int gemv_q8(const int8_t* A, const uint16_t* scale, const uint16_t* x, float* y, int M, int N,
            hipStream_t stream)
{
    return gemv::launch(gemv::kQ8, A, scale, x, y, M, N, stream);
}

int gemv_q4(const uint8_t* A, const uint16_t* scale, const uint16_t* x, float* y, int M, int N,
            hipStream_t stream)
{
    return gemv::launch(gemv::kQ4, A, scale, x, y, M, N, stream);
}

const char* gemv_status_string(int status)
{
    switch (status) {
    case GEMV_OK: return "ok";
    case GEMV_E_INVAL: return "invalid argument";
    case GEMV_E_UNSUPPORTED: return "unsupported shape for this format";
    case GEMV_E_LAUNCH: return "kernel launch failed";
    case GEMV_E_DEVICE: return "no usable HIP device";
    default: return "unknown status";
    }
}

int gemv_probe_read(const void* buf, size_t bytes, uint32_t* sink, uint32_t guard, hipStream_t stream)
{
    if (bytes % 16 != 0 || (bytes > 0 && (buf == nullptr || !gemv::aligned16(buf))) || sink == nullptr)
        return GEMV_E_INVAL;
    if (bytes == 0)
        return GEMV_OK;
    const int64_t n16 = (int64_t)(bytes / 16);
    int grid = 0;
    if (int rc = gemv::probe_grid(n16, &grid); rc != GEMV_OK)
        return rc;
    const gemv::u32x4* b = static_cast<const gemv::u32x4*>(buf);
    void* args[] = {(void*)&b, (void*)&n16, (void*)&sink, (void*)&guard};
    const hipError_t err = hipLaunchKernel(
        reinterpret_cast<const void*>(&gemv::probe_read_kernel<gemv::kProbeU, gemv::kNT>), dim3(grid),
        dim3(256), args, 0, stream);
    return err == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}

int gemv_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream)
{
    if (bytes % 16 != 0)
        return GEMV_E_INVAL;
    if (bytes == 0)
        return GEMV_OK;
    if (src == nullptr || dst == nullptr || !gemv::aligned16(src) || !gemv::aligned16(dst))
        return GEMV_E_INVAL;
    const int64_t n16 = (int64_t)(bytes / 16);
    int grid = 0;
    if (int rc = gemv::probe_grid(n16, &grid); rc != GEMV_OK)
        return rc;
    const gemv::u32x4* s = static_cast<const gemv::u32x4*>(src);
    gemv::u32x4* d = static_cast<gemv::u32x4*>(dst);
    void* args[] = {(void*)&s, (void*)&d, (void*)&n16};
    const hipError_t err = hipLaunchKernel(
        reinterpret_cast<const void*>(&gemv::probe_copy_kernel<gemv::kProbeU, gemv::kNT>), dim3(grid),
        dim3(256), args, 0, stream);
    return err == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}

}  // extern "C"

namespace gemv {
namespace {

// The report of plan p for a call of M x N.
void info_of_plan(int kind, int M, int N, const Plan& p, gemv_launch_info* info)
{
    info->variant = p.variant;
    info->grid = p.grid;
    info->block = p.block;
    const int64_t waves = (int64_t)p.grid * p.waves;
    if (p.variant == 4) {
        // row groups of 64 / L rows, walked grid-stride by the waves
        const int64_t R = packed_rows_per_load(N / elems_per_chunk(kind));
        const int64_t groups = ((int64_t)M + R - 1) / R;
        info->rows_per_wave = waves > 0 ? (int)((groups + waves - 1) / waves * R) : 0;
    } else if (p.variant == 7) {
        // R rows of every slab the workgroup takes
        const int64_t slabs = ((int64_t)M + p.rows - 1) / p.rows;
        info->rows_per_wave = p.grid > 0 ? (int)((slabs + p.grid - 1) / p.grid * p.rows) : 0;
    } else {
        info->rows_per_wave = waves > 0 ? (int)(((int64_t)M + waves - 1) / waves) : 0;
    }
    info->units_in_flight = p.D;
    info->lds_bytes = p.lds;
    info->stage_order = p.variant == 1 ? p.stg : -1;
}

// gemv_describe_launch's report for a device of `dev`'s properties.
void fill_launch_info(int kind, int M, int N, bool aligned, const Device& dev, gemv_launch_info* info)
{
    info_of_plan(kind, M, N, make_plan(kind, M, N, aligned, dev), info);
}

// An explicit plan (gemv_plan) checked against the kernels the library holds
// and the shape, completed to a launch as the planner's plans are; GEMV_OK,
// GEMV_E_INVAL or GEMV_E_UNSUPPORTED.
int plan_from_user(int kind, int M, int N, const Device& dev, const gemv_plan& u, Plan* out)
{
    if (kind < 0 || kind > 5 || M < 1 || N < 1)
        return GEMV_E_INVAL;
    if (kind == kQ4 && N % 128 != 0)
        return GEMV_E_UNSUPPORTED;
    const int epc = elems_per_chunk(kind);
    // the bandwidth path only (rows_plan's conditions for the element-wise kernel)
    if (N % epc != 0 || (int64_t)(N / epc) * 16 >= ((int64_t)1 << 31) || M > (1 << 30))
        return GEMV_E_UNSUPPORTED;
    const int nchunks = N / epc;
    const int P = (nchunks + 63) / 64;
    const bool fp = kind == kF32 || kind == kF16 || kind == kF16H;
    const bool intk = kind == kQ8 || kind == kQ4;
    Plan p{};
    p.variant = u.variant;
    p.waves = u.waves;
    p.D = u.units_in_flight;
    p.rows = u.rows_per_wave;
    p.stg = u.stage_order;
    p.cap = u.cap;
    if (p.rows < 1 || p.cap < 0)
        return GEMV_E_UNSUPPORTED;
    switch (p.variant) {
    case 1:
    case 2: {
        const bool staged = p.variant == 1;
        if (staged ? (fp || p.stg < 0 || p.stg > 2) : p.stg != -1)
            return GEMV_E_UNSUPPORTED;   // FP32/FP16 read x with each unit
        const bool common = (p.waves == 4 || p.waves == 8) && (p.D == 2 || p.D == 4 || p.D == 8);
        // the depths instantiated for rows of 5 and 6 units
        const bool d5 = staged && p.waves == 4 && p.D == 5 &&
                        ((kind == kQ8 && p.stg == 2) || (kind == kQ4 && p.stg == 1));
        const bool d3 = staged && p.waves == 4 && p.D == 3 && kind == kQ4 && p.stg == 1;
        if (!(common || d5 || d3))
            return GEMV_E_UNSUPPORTED;
        if (staged) {
            const int64_t lds = lds_bytes(kind, nchunks) + (p.stg == 2 ? kSplitSpareBytes : 0);
            if (lds > dev.lds_max)
                return GEMV_E_UNSUPPORTED;
            p.lds = (int)lds;
        }
        finish_rows(M, dev.cus, &p);
        break;
    }
    case 4: {
        if (!intk || nchunks > kPackedMaxChunks || p.waves != 8 || (p.D != 1 && p.D != 2) || p.stg != -1)
            return GEMV_E_UNSUPPORTED;
        const int R = packed_rows_per_load(nchunks);
        const int64_t groups = ((int64_t)M + R - 1) / R;
        p.block = p.waves * 64;
        const int64_t waves_needed = (groups + p.rows - 1) / p.rows;
        int64_t grid = (waves_needed + p.waves - 1) / p.waves;
        if (p.cap > 0 && grid > (int64_t)p.cap * dev.cus)
            grid = (int64_t)p.cap * dev.cus;
        p.grid = gemv_device::capped_grid(grid, p.block);
        break;
    }
    case 5: {
        if (P > 3 || p.stg != -1)
            return GEMV_E_UNSUPPORTED;
        p.xk = P;
        const bool ok = P == 3   ? p.D == 3 && (p.waves == 4 || p.waves == 8)
                        : P == 2 ? p.D == 2 && p.waves == 4
                                 : (p.D == 1 || p.D == 2) && (p.waves == 4 || p.waves == 8);
        if (!ok)
            return GEMV_E_UNSUPPORTED;
        finish_rows(M, dev.cus, &p);
        break;
    }
    case 6: {
        const int S = p.waves;
        if (kind == kF16H || p.stg != -1 || p.cap != 0 || p.rows != 1 || !(S == 2 || S == 4 || S == 8 || S == 16) ||
            2 * S > P || !(p.D == 2 || p.D == 4) || (int64_t)M * S * 64 > gemv_device::kMaxWorkItems)
            return GEMV_E_UNSUPPORTED;
        p.xk = S;
        p.block = S * 64;
        p.grid = M;
        break;
    }
    case 7: {
        // S = waves waves per slab, Q = P / S passes per wave (1 or 2)
        const int S = p.waves;
        if (!(kind == kQ8 || kind == kQ4 || kind == kF16X32) || p.stg != -1 || S < 1 || S > 16 || P % S != 0 ||
            P / S > 2 || !(p.D == 4 || p.D == 8) || !(p.rows == 4 || p.rows == 8) || p.rows * (P / S) % p.D != 0)
            return GEMV_E_UNSUPPORTED;
        p.xk = P / S;
        p.block = S * 64;
        p.lds = 0;
        int64_t grid = ((int64_t)M + p.rows - 1) / p.rows;
        if (p.cap > 0 && grid > (int64_t)p.cap * dev.cus)
            grid = (int64_t)p.cap * dev.cus;
        p.grid = gemv_device::capped_grid(grid, p.block);
        break;
    }
    default:
        return GEMV_E_UNSUPPORTED;
    }
    *out = p;
    return GEMV_OK;
}

int check_describe(int kind, int M, int N, const gemv_launch_info* info)
{
    if (info == nullptr || kind < 0 || kind > 5 || M < 0 || N < 0)
        return GEMV_E_INVAL;
    if (kind == kQ4 && N % 128 != 0)
        return GEMV_E_UNSUPPORTED;
    return GEMV_OK;
}

}  // namespace
}  // namespace gemv

extern "C" {

int gemv_describe_launch(int kind, int M, int N, int aligned, gemv_launch_info* info)
{
    if (int rc = gemv::check_describe(kind, M, N, info); rc != GEMV_OK)
        return rc;
    gemv::Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    gemv::fill_launch_info(kind, M, N, aligned != 0, dev, info);
    return GEMV_OK;
}

int gemv_describe_launch_for(int kind, int M, int N, int aligned, int cus, int lds_max, gemv_launch_info* info)
{
    if (int rc = gemv::check_describe(kind, M, N, info); rc != GEMV_OK)
        return rc;
    if (cus <= 0 || lds_max <= 0)
        return GEMV_E_INVAL;
    gemv::fill_launch_info(kind, M, N, aligned != 0, gemv::Device{cus, lds_max}, info);
    return GEMV_OK;
}

int gemv_check_plan_for(int kind, int M, int N, int cus, int lds_max, const gemv_plan* plan, gemv_launch_info* info)
{
    if (plan == nullptr || info == nullptr || cus <= 0 || lds_max <= 0)
        return GEMV_E_INVAL;
    gemv::Plan p{};
    if (int rc = gemv::plan_from_user(kind, M, N, gemv::Device{cus, lds_max}, *plan, &p); rc != GEMV_OK)
        return rc;
    gemv::info_of_plan(kind, M, N, p, info);
    return GEMV_OK;
}

int gemv_launch_plan(int kind, const void* A, const uint16_t* scale, const void* x, float* y, int M, int N,
                     const gemv_plan* plan, hipStream_t stream)
{
    if (plan == nullptr || A == nullptr || x == nullptr || y == nullptr ||
        ((kind == gemv::kQ8 || kind == gemv::kQ4) && scale == nullptr))
        return GEMV_E_INVAL;
    if (!gemv::aligned16(A) || !gemv::aligned16(x))
        return GEMV_E_INVAL;
    gemv::Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    gemv::Plan p{};
    if (int rc = gemv::plan_from_user(kind, M, N, dev, *plan, &p); rc != GEMV_OK)
        return rc;
    return gemv::launch_planned(kind, p, A, scale, x, y, M, N, stream);
}

}  // extern "C"
