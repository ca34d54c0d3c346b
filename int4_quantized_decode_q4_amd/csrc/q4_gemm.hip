// q4_gemm.hip -- batched form of the int4 dequantizing matmul.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_geometry.h"
#include "q4_internal.h"

namespace q4 {

hipError_t launch_gemm(const Geometry &geo, const void *wdata, const uint16_t *X, int64_t m,
                       int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    // batched form, one GEMV launch per activation row (replaced by the
    // VALU multi-vector and MFMA kernels)
    for (int64_t i = 0; i < m; ++i) {
        const hipError_t e = launch_gemv_family(geo, EPI_F16, wdata, X + i * k, Y + i * n, n, k, n,
                                                ArgmaxScratch{nullptr, nullptr}, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace q4
