/*
 * gemv.h -- C ABI of the MI355X (gfx950) row-major GEMV library.
 *
 *     y[M] = A[M, N] . x[N],   y_i = sum_j A_ij x_j
 *
 * The operation is the plain matrix-vector product ("Making GEMV Fast",
 * section "Algorithm"; the llama.cpp FP16 GEMV walkthrough, opening
 * equation), with A dense and row-major: element (i, j) at linear offset
 * i*N + j, leading dimension N, no stride argument ("Making GEMV Fast",
 * section "Row-major indexing refresher").  Four storage formats for A, with
 * binary16 or (for FP16 A) FP32 x; every entry point but the lossy
 * gemv_f16_acc16 accumulates in FP32, and all write FP32 y.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Pointers   Device pointers (hipMalloc'd or any device-accessible
 *              allocation).  The caller owns every buffer.  The library
 *              allocates nothing, keeps no pointer after returning, and needs
 *              no workspace.
 *   Binary16   FP16 values (x, FP16 A, scales) are passed as IEEE 754
 *              binary16 bit patterns in uint16_t.  Subnormals are honoured.
 *   Stream     Work is enqueued on `stream` (0 = the null stream) and the
 *              call returns without synchronising; y is valid once the
 *              caller synchronises that stream.
 *   Semantics  y is overwritten (no alpha/beta, no accumulation into y).
 *              N == 0 writes y = 0 (the empty sum).  M == 0 is a no-op.
 *   Aliasing   y must not overlap A, x or scale.
 *   Alignment  Each pointer needs only its element's natural alignment
 *              (4 bytes for float, 2 for binary16, 1 for int8/uint8).  The
 *              bandwidth path needs 16-byte-aligned A and x and a row length
 *              in bytes that is a multiple of 16; other inputs take a slower
 *              element-wise path.
 *   Results    Deterministic: the reduction order depends only on (format,
 *              M, N, pointer alignment, device), so repeated calls give
 *              bitwise identical y.  No atomics.
 *   Errors     Every entry point returns a gemv_status and never prints or
 *              exits.  Invalid arguments are rejected before anything is
 *              enqueued.  Faults during execution surface at the caller's
 *              next synchronisation, as for any HIP kernel.
 *   Threads    Entry points are thread-safe and may be called concurrently on
 *              different streams.  The only state the library keeps is each
 *              device's compute-unit count and LDS per workgroup, read on its
 *              first call on that device (under a lock) and kept until the
 *              process ends; the launch geometry is chosen from them.
 */
#ifndef MBGR_GEMV_H
#define MBGR_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same typedef as the HIP runtime header, so that C callers need no HIP headers. */
typedef struct ihipStream_t* hipStream_t;

typedef enum gemv_status {
    GEMV_OK = 0,
    GEMV_E_INVAL = 1,       /* negative M or N, or a null pointer where data is needed */
    GEMV_E_UNSUPPORTED = 2, /* format constraint violated (INT4: N % 128 != 0)        */
    GEMV_E_LAUNCH = 3,      /* the HIP runtime refused the kernel launch             */
    GEMV_E_DEVICE = 4       /* no current HIP device or its properties are unreadable */
} gemv_status;

/* FP32: A float[M*N] row-major, x float[N], y float[M].
 * ("cuda-gemv-optimization", section "Results": FP32 row-major GEMV.) */
int gemv_f32(const float* A, const float* x, float* y, int M, int N, hipStream_t stream);

/* FP16 weights and activations, FP32 accumulation and output:
 * A binary16[M*N] row-major, x binary16[N], y float[M].
 * (llama.cpp FP16 GEMV walkthrough: FP16 weight and hidden state, FP32
 * accumulation and output; "membound", section "Results".) */
int gemv_f16(const uint16_t* A, const uint16_t* x, float* y, int M, int N, hipStream_t stream);

/* FP16 weights with an FP32 hidden state, FP32 accumulation and output:
 *   A binary16[M*N] row-major, x float[N], y float[M].
 * Each weight is widened to FP32 exactly and multiplied by x_j exactly, so
 * only the FP32 additions round, as in gemv_f32.  x takes 4N bytes against
 * gemv_f16's 2N; A's traffic is the same.
 * (llama.cpp FP16 GEMV walkthrough, implementation note: the original
 * kernel keeps the hidden state in FP32.) */
int gemv_f16x32(const uint16_t* A, const float* x, float* y, int M, int N, hipStream_t stream);

/* FP16 weights and activations with FP16 ACCUMULATION -- LOSSY:
 *   A binary16[M*N] row-major, x binary16[N], y float[M].
 * Each lane of the kernel keeps its running sums in binary16 (one rounding
 * to binary16 per term, at most k = max(ceil(N/64), 4) terms per sum); only
 * the final cross-lane reduction and y are FP32.  For every row,
 *   |y_i - sum_j A_ij x_j| <= ((1 + g16(k)) (1 + g32(8)) - 1) * sum_j |A_ij x_j|
 *                             + N * 2^-24,
 * with gB(k) = k*uB / (1 - k*uB), u16 = 2^-11, u32 = 2^-24 (the N*2^-24
 * term covers roundings of sums in binary16's subnormal range, spacing
 * 2^-24).  A partial sum beyond binary16's
 * range (65504) gives an infinite y_i.  Use gemv_f16 unless this rounding is
 * acceptable.
 * (llama.cpp FP16 GEMV walkthrough, implementation note: the original
 * kernel can accumulate in FP16 or FP32.) */
int gemv_f16_acc16(const uint16_t* A, const uint16_t* x, float* y, int M, int N, hipStream_t stream);

/* INT8 weights with one symmetric binary16 scale per row:
 *   A int8[M*N] row-major, scale binary16[M], x binary16[N], y float[M],
 *   y_i = sum_j (A_ij * scale_i) * x_j.
 * Every int8 value, -128 included, is accepted.
 * ("membound", section "The kernel decode actually runs: dequant GEMV".) */
int gemv_q8(const int8_t* A, const uint16_t* scale, const uint16_t* x, float* y, int M, int N,
            hipStream_t stream);

/* INT4 weights, two per byte, with one symmetric binary16 scale per row and
 * 128-column group:
 *   A uint8[M*(N/2)] row-major; byte (i, k) holds column 2k in its low
 *     nibble and column 2k+1 in its high nibble, each a two's-complement
 *     value in [-8, 7];
 *   scale binary16[M*(N/128)] row-major, scale[i*(N/128) + j/128] covers
 *     columns j of row i;
 *   x binary16[N], y float[M],
 *   y_i = sum_j (q_ij * scale_{i, j/128}) * x_j.
 * N must be a multiple of 128 (GEMV_E_UNSUPPORTED otherwise).
 * ("membound", section "The kernel decode actually runs: dequant GEMV":
 * symmetric per-group-of-128 scales.) */
int gemv_q4(const uint8_t* A, const uint16_t* scale, const uint16_t* x, float* y, int M, int N,
            hipStream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* gemv_status_string(int status);

/* ---- measurement kernels --------------------------------------------------
 * The pages measure a GEMV against the bandwidth a plain stream achieves on
 * the same device in the same run: a pure-read probe is the denominator for
 * GEMV's read-dominated traffic, a streaming copy for balanced read+write
 * traffic ("membound", section "Why GEMV, and why MBU").  These are those
 * probes; they are not part of the GEMV computation.
 */

/* Reads `bytes` bytes of `buf` once with 16-byte loads.  `bytes` must be a
 * multiple of 16 and `buf` 16-byte aligned (GEMV_E_INVAL otherwise).  The
 * loaded words are XOR-folded; the fold is written to `sink[0]` only if it
 * equals `guard`, so the reads cannot be optimised away and nothing is
 * normally written.  `sink` must point to at least 4 writable bytes. */
int gemv_probe_read(const void* buf, size_t bytes, uint32_t* sink, uint32_t guard, hipStream_t stream);

/* Copies `bytes` bytes from `src` to `dst` with 16-byte loads and stores.
 * Same size and alignment rules; the buffers must not overlap. */
int gemv_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Launch geometry the library uses for a call.  kind: 0 f32, 1 f16, 2 q8,
 * 3 q4, 4 f16x32 (FP16 A, FP32 x), 5 f16_acc16 (FP16 accumulation).
 * `aligned` states whether A and x are 16-byte aligned.  Fills `info` with
 * the variant (1 = streaming kernel with x staged in LDS, 2 = streaming
 * kernel with x read from global memory, 3 = element-wise kernel, 4 = packed
 * kernel for INT8/INT4 rows of at most 32 16-byte chunks, several rows per
 * wave load, 5 = kernel for rows of one to three wave loads with each
 * lane's x in registers, 6 = split rows: few long rows, a workgroup of 2 to
 * 16 waves per row whose wave sums meet in LDS, 7 = row slabs: INT8, INT4
 * and FP16 with FP32 x, a workgroup of S waves takes 4 or 8 rows at a time,
 * each wave one or two passes of every row with its slice of x in
 * registers, the wave sums of a row meeting in LDS), grid and workgroup
 * sizes, rows per wave (at most; row slabs: the rows each workgroup takes),
 * 1-KiB loads in flight per wave, dynamic LDS bytes (x staged up to what
 * one workgroup may hold on the device), and the order in which x is staged
 * relative to the first loads of A.  The geometry is chosen per shape:
 * workgroups of 2 to 16 waves, 1 to 8 loads in flight, 1 to 4 rows (packed:
 * row groups) per wave, more where a grid cap makes waves walk further --
 * every launch keeps grid x block at or below 2^30 work-items (the llama.cpp
 * walkthrough's implementation note: the original kernel selects its block
 * size at run time).  Returns GEMV_OK or an error code; it reads the current
 * device's compute-unit count and LDS per workgroup and launches nothing. */
typedef struct gemv_launch_info {
    int variant;
    int grid;
    int block;
    int rows_per_wave;
    int units_in_flight;
    int lds_bytes;
    int stage_order;   /* variant 1: 0 A first, 1 x first, 2 x loads / A / x writes; else -1 */
} gemv_launch_info;

int gemv_describe_launch(int kind, int M, int N, int aligned, gemv_launch_info* info);

/* The same report for a device with `cus` compute units whose workgroups may
 * hold `lds_max` bytes of LDS (MI355X: 256 and 163840), without touching
 * any device: for planning, and for testing the geometry rules on a host
 * without a GPU.  GEMV_E_INVAL also for cus <= 0 or lds_max <= 0. */
int gemv_describe_launch_for(int kind, int M, int N, int aligned, int cus, int lds_max, gemv_launch_info* info);

/* An explicit launch plan, for plan searches and tuning: the choices the
 * planner makes for a call (the llama.cpp walkthrough's implementation note:
 * the block size is chosen at run time; here every choice can also be
 * given).
 *   variant          1 streaming kernel, x staged in LDS (INT8, INT4, FP16
 *                    with FP32 x); 2 streaming kernel, x read with each
 *                    unit; 4 packed short rows (INT8/INT4 rows of at most
 *                    32 16-byte chunks); 5 x in registers (rows of exactly
 *                    1-3 wave loads); 6 split rows (a workgroup per row);
 *                    7 row slabs (INT8, INT4, FP16 with FP32 x: S waves own
 *                    P / S = 1 or 2 passes each of every row, P the wave
 *                    loads per row, S <= 16)
 *   waves            waves per workgroup (split rows: waves per row, 2-16;
 *                    row slabs: S)
 *   units_in_flight  1-KiB wave loads in flight per wave (row slabs: 4 or 8,
 *                    dividing the slab's units per wave)
 *   rows_per_wave    rows (packed: row groups) per wave the grid is sized
 *                    for; waves walk whatever rows lie beyond (1 for split;
 *                    row slabs: rows per slab, 4 or 8)
 *   stage_order      variant 1: 0 A's first loads before x's staging, 1 x
 *                    first, 2 staging loads / A's first loads / LDS writes;
 *                    -1 otherwise
 *   cap              at most this many workgroups per CU (0: no cap)
 * Only combinations the library holds a kernel for are accepted. */
typedef struct gemv_plan {
    int variant;
    int waves;
    int units_in_flight;
    int rows_per_wave;
    int stage_order;
    int cap;
} gemv_plan;

/* Whether `plan` can run `kind` at M x N on a device with `cus` compute
 * units and `lds_max` bytes of LDS per workgroup, touching no device: fills
 * `info` with the launch it makes and returns GEMV_OK, or returns
 * GEMV_E_UNSUPPORTED for a plan the library holds no kernel for or that does
 * not fit the shape (a staged x beyond lds_max, x in registers for rows not
 * of 1-3 wave loads, split rows with fewer than two loads per wave or beyond
 * 2^30 work-items, packed rows for FP formats or rows over 32 chunks, row
 * slabs for FP32/FP16 or with S not dividing P into one or two passes, FP16
 * accumulation outside variants 2 and 5), GEMV_E_INVAL for bad arguments
 * (kind outside 0-5, M or N < 1, cus or lds_max <= 0, null pointers).  The
 * shape must take the bandwidth path (N a multiple of a 16-byte chunk's
 * elements, rows under 2 GiB, at most 2^30 rows). */
int gemv_check_plan_for(int kind, int M, int N, int cus, int lds_max, const gemv_plan* plan,
                        gemv_launch_info* info);

/* Runs the GEMV of `kind` (operands as for gemv_f32 ... gemv_q4; `scale`
 * ignored for FP formats) with `plan` instead of the planner's choice, on
 * the current device; y is the same up to the summation order the plan
 * implies (bit for bit where it sums each lane's chunks as the planner's
 * plan does).  Checks as gemv_check_plan_for, plus GEMV_E_INVAL for A or x
 * not 16-byte aligned.  Enqueues on `stream` and returns; GEMV_E_LAUNCH if
 * the launch fails. */
int gemv_launch_plan(int kind, const void* A, const uint16_t* scale, const void* x, float* y, int M, int N,
                     const gemv_plan* plan, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MBGR_GEMV_H */
