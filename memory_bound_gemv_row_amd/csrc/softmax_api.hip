// softmax_api.hip -- C ABI of the row softmax (declared in
// include/gemv_softmax.h): validation, geometry and launch.
#include "gemv_softmax.h"
#include "softmax_kernels.hpp"

#include <hip/hip_runtime.h>

#include <mutex>

namespace gsoftmax {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kWavesPerCu = 32;   // resident waves a CU can hold
std::mutex g_mutex;
int g_cus[kMaxDevices] = {0};

int cu_count(int* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMV_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return GEMV_E_DEVICE;
        g_cus[dev] = n;
    }
    *out = g_cus[dev];
    return GEMV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Waves per row and units held per wave, so that a row of P units stays in
// registers up to 256 units (131072 columns) with at most 64 VGPRs of data.
void geometry(int P, int* waves, int* upw)
{
    if (P <= 16) { *waves = 4; *upw = 4; }
    else if (P <= 32) { *waves = 4; *upw = 8; }
    else if (P <= 64) { *waves = 8; *upw = 8; }
    else if (P <= 128) { *waves = 8; *upw = 16; }
    else { *waves = 16; *upw = 16; }
}

const void* kernel_for(int waves, int upw)
{
    if (waves == 4)
        return upw == 4 ? reinterpret_cast<const void*>(&softmax_f16_kernel<4, 4>)
                        : reinterpret_cast<const void*>(&softmax_f16_kernel<4, 8>);
    if (waves == 8)
        return upw == 8 ? reinterpret_cast<const void*>(&softmax_f16_kernel<8, 8>)
                        : reinterpret_cast<const void*>(&softmax_f16_kernel<8, 16>);
    return reinterpret_cast<const void*>(&softmax_f16_kernel<16, 16>);
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
        const unsigned grid4 = (unsigned)(((int64_t)M + 3) / 4);
        err = hipLaunchKernel(reinterpret_cast<const void*>(&softmax_f16_elementwise), dim3(grid4), dim3(256), args,
                              0, stream);
    } else {
        int waves = 4, upw = 4;
        geometry((N / 8 + 63) / 64, &waves, &upw);
        const int per_cu = kWavesPerCu / waves;
        const int grid = M < cus * per_cu ? M : cus * per_cu;
        err = hipLaunchKernel(kernel_for(waves, upw), dim3(grid), dim3(waves * 64), args, 0, stream);
    }
    return err == hipSuccess ? GEMV_OK : GEMV_E_LAUNCH;
}
