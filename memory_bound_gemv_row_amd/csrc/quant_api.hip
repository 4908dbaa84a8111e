// quant_api.hip -- C ABI of the weight quantiser (declared in
// include/gemv_quant.h): validation, geometry and launch.
#include "gemv_quant.h"
#include "device_info.hpp"
#include "quant_kernels.hpp"

#include <hip/hip_runtime.h>

namespace gquant {
namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int launch(const void* fn, int grid, int block, const float* W, void* q, uint16_t* scale, float* row_sse, int M,
           int N, hipStream_t stream)
{
    void* args[] = {(void*)&W, (void*)&q, (void*)&scale, (void*)&row_sse, (void*)&M, (void*)&N};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, stream) == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}

// INT8 kernel for rows of P units and its waves per workgroup: 4 waves of 4
// units up to 16 units, 8 of 4 up to 32, 8 of 8 beyond (rows of more than 64
// units are read twice).  Graph-timed A/B with a workgroup per row against
// 4 waves and rows walked by 8 workgroups per CU: 16384x2048 34.0 -> 31.3 us,
// 14336x4096 52.5 -> 48.2, 8192x6144 45.5 -> 43.6, 8192x8192 58.3 -> 56.3,
// 4096x14336 57.9 -> 51.8, 4096x16384 65.6 -> 59.2, 2048x32768 101.9 -> 97.9.
template <bool SSE>
const void* q8_kernel(int P, int* waves)
{
    *waves = P <= 16 ? 4 : 8;
    return P <= 16 ? reinterpret_cast<const void*>(&quantize_q8_kernel<4, 4, SSE>)
         : P <= 32 ? reinterpret_cast<const void*>(&quantize_q8_kernel<8, 4, SSE>)
                   : reinterpret_cast<const void*>(&quantize_q8_kernel<8, 8, SSE>);
}

template <bool SSE>
const void* row_kernel_q4_sse(int waves)
{
    return waves == 2 ? reinterpret_cast<const void*>(&quantize_q4_rows_kernel<2, 4, SSE>)
         : waves == 4 ? reinterpret_cast<const void*>(&quantize_q4_rows_kernel<4, 4, SSE>)
         : waves == 8 ? reinterpret_cast<const void*>(&quantize_q4_rows_kernel<8, 4, SSE>)
                      : reinterpret_cast<const void*>(&quantize_q4_rows_kernel<16, 4, SSE>);
}

const void* row_kernel_q4(int waves, bool sse)
{
    return sse ? row_kernel_q4_sse<true>(waves) : row_kernel_q4_sse<false>(waves);
}

int check(const float* W, const void* q, const uint16_t* scale, int M, int N)
{
    if (M < 0 || N < 0)
        return GEMV_E_INVAL;
    if (M > 0 && (scale == nullptr || (N > 0 && (W == nullptr || q == nullptr))))
        return GEMV_E_INVAL;
    return GEMV_OK;
}

}  // namespace
}  // namespace gquant

extern "C" {

int gemv_quantize_q8(const float* W, int8_t* q, uint16_t* scale, float* row_sse, int M, int N,
                     hipStream_t stream)
{
    using namespace gquant;
    if (int rc = check(W, q, scale, M, N); rc != GEMV_OK)
        return rc;
    if (M == 0)
        return GEMV_OK;
    // the grids need no CU count, but a call without a usable device fails
    // here like the others
    gemv_device::Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    // more than 2^30 rows: the row-walking kernels' int row cursors could
    // pass INT_MAX; the element-wise kernel indexes rows in 64 bits
    const int grid4 = gemv_device::capped_grid(((int64_t)M + 3) / 4, 256);
    if (N == 0 || N % 4 != 0 || !aligned(W, 16) || !aligned(q, 4) || M > (1 << 30))
        return launch(reinterpret_cast<const void*>(&quantize_elementwise_kernel<127>), grid4, 256, W, q, scale,
                      row_sse, M, N, stream);
    // a workgroup per row; units per wave sized so that rows up to 64 units
    // (N <= 16384) stay in registers
    const int P = (N / 4 + 63) / 64;
    int waves = 4;
    const void* fn = row_sse != nullptr ? q8_kernel<true>(P, &waves) : q8_kernel<false>(P, &waves);
    return launch(fn, gemv_device::capped_grid(M, waves * 64), waves * 64, W, q, scale, row_sse, M, N, stream);
}

int gemv_quantize_q4(const float* W, uint8_t* q, uint16_t* scale, float* row_sse, int M, int N,
                     hipStream_t stream)
{
    using namespace gquant;
    if (int rc = check(W, q, scale, M, N); rc != GEMV_OK)
        return rc;
    if (N % 128 != 0)
        return GEMV_E_UNSUPPORTED;
    if (M == 0)
        return GEMV_OK;
    // the grids need no CU count, but a call without a usable device fails
    // here like the others
    gemv_device::Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    const int grid4 = gemv_device::capped_grid(((int64_t)M + 3) / 4, 256);
    if (N == 0 || !aligned(W, 16) || !aligned(q, 2) || M > (1 << 30))   // as for INT8
        return launch(reinterpret_cast<const void*>(&quantize_elementwise_kernel<7>), grid4, 256, W, q, scale,
                      row_sse, M, N, stream);
    const int P = (N / 4 + 63) / 64;
    if (P <= 4) {
        // one wave per row, 4 waves per workgroup, 4 units in flight per wave
        const void* fn = row_sse != nullptr ? reinterpret_cast<const void*>(&quantize_q4_kernel<4, 4, true>)
                                            : reinterpret_cast<const void*>(&quantize_q4_kernel<4, 4, false>);
        return launch(fn, grid4, 256, W, q, scale, row_sse, M, N, stream);
    }
    // a workgroup per row, 4 units in flight per wave, 2 to 16 waves so that
    // each takes about 3 to 8 of the row's units (a wave per row pads rows
    // of 5-15 units to a multiple of 4: 16384 x 1536 27.5 -> 22.6 us,
    // 32768 x 1280 49.4 -> 36.2, 16384 x 3584 55.4 -> 45.6)
    const int waves = P < 12 ? 2 : (P < 48 ? 4 : (P < 128 ? 8 : 16));
    return launch(row_kernel_q4(waves, row_sse != nullptr), gemv_device::capped_grid(M, waves * 64), waves * 64, W, q,
                  scale, row_sse, M, N, stream);
}

}  // extern "C"
