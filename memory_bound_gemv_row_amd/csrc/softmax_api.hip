// softmax_api.hip -- C ABI of the row softmax (declared in
// include/gemv_softmax.h): validation, geometry and launch.
#include "gemv_softmax.h"
#include "device_info.hpp"
#include "softmax_kernels.hpp"

#include <hip/hip_runtime.h>

namespace gsoftmax {
namespace {

// compute units of the current device
int cu_count(int* out)
{
    gemv_device::Device dev{};
    if (int rc = gemv_device::current(&dev); rc != GEMV_OK)
        return rc;
    *out = dev.cus;
    return GEMV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Geometry for rows of P units: waves per row and units held per wave, so
// that a row stays in registers up to 256 units (131072 columns) with at
// most 64 VGPRs of data; whether a workgroup loads its next row while it
// stores the current one; and for those, workgroups per CU.  The prefetch and the deeper
// grids for 4-wave rows were measured (graph-timed, rotating buffers):
// 8192 x 8192 47.4 -> 46.3 us, 4096 x 32768 98.2 -> 94.0, 16384 x 4096
// 61.7 -> 57.7; with 16 units per wave (rows over 64 units) the prefetch
// was slower (2048 x 65536 98.9 -> 109.4) and stays off.
struct Geometry {
    int waves, upw, per_cu;
    bool prefetch;
};

Geometry geometry(int P)
{
    if (P <= 16) return {4, 4, 16, true};
    if (P <= 32) return {4, 8, 16, true};
    if (P <= 64) return {8, 8, 3, true};
    if (P <= 128) return {8, 16, 0, false};   // a workgroup per row (per_cu unused)
    return {16, 16, 0, false};
}

const void* kernel_for(const Geometry& g)
{
    if (g.waves == 4)
        return g.upw == 4 ? reinterpret_cast<const void*>(&softmax_f16_kernel<4, 4, true>)
                          : reinterpret_cast<const void*>(&softmax_f16_kernel<4, 8, true>);
    if (g.waves == 8)
        return g.upw == 8 ? reinterpret_cast<const void*>(&softmax_f16_kernel<8, 8, true>)
                          : reinterpret_cast<const void*>(&softmax_f16_kernel<8, 16, false>);
    return reinterpret_cast<const void*>(&softmax_f16_kernel<16, 16, false>);
}

}  // namespace
}  // namespace gsoftmax

extern "C" int gemv_softmax_f16(const uint16_t* x, uint16_t* y, int M, int N, hipStream_t stream)
{
    using namespace gsoftmax;
    if (M < 0 || N < 0)
        return GEMV_E_INVAL;
    if (M == 0 || N == 0)
        return GEMV_OK;
    if (x == nullptr || y == nullptr)
        return GEMV_E_INVAL;
    int cus = 0;
    if (int rc = cu_count(&cus); rc != GEMV_OK)
        return rc;
    void* args[] = {(void*)&x, (void*)&y, (void*)&M, (void*)&N};
    hipError_t err;
    // more than 2^30 rows: the row-per-workgroup kernel's int row cursor
    // could pass INT_MAX; the element-wise kernel indexes rows in 64 bits
    if (N % 8 != 0 || !aligned16(x) || !aligned16(y) || M > (1 << 30)) {
        const int grid4 = gemv_device::capped_grid(((int64_t)M + 3) / 4, 256);
        err = hipLaunchKernel(reinterpret_cast<const void*>(&softmax_f16_elementwise), dim3(grid4), dim3(256), args,
                              0, stream);
    } else {
        // rows that reload the next row walk a grid of per_cu workgroups per
        // CU; the others take a workgroup per row (2048 x 65536 99.5 ->
        // 98.0 us, 1024 x 131072 107.3 -> 106.6 against walking)
        const Geometry g = geometry((N / 8 + 63) / 64);
        const int grid = !g.prefetch ? gemv_device::capped_grid(M, g.waves * 64)
                                     : (M < cus * g.per_cu ? M : cus * g.per_cu);
        err = hipLaunchKernel(kernel_for(g), dim3(grid), dim3(g.waves * 64), args, 0, stream);
    }
    return err == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}
