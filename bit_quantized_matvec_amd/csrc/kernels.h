// kernels.h -- host-side launchers of the HIP kernels (internal to libtq).
// Arguments are validated by the C-ABI layer before any launcher runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace tq {

hipError_t launch_quantize_q8k(const float* x, int64_t nblocks, int8_t* q, float* d, int16_t* bsums, hipStream_t s);

hipError_t launch_repack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, int32_t* bad_flag, hipStream_t s);
hipError_t launch_unrepack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);
hipError_t launch_repack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);
hipError_t launch_unrepack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);

// y[rows] (fp32) or, if idots != nullptr, the int32 group dots [rows][G].
hipError_t launch_gemv_pq2(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s);
hipError_t launch_gemv_ptq1(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx,
                            const int16_t* bsums, float* y, int32_t* idots, hipStream_t s);
// y[tokens][rows] or idots [tokens][rows][G].
hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                           float* y, int32_t* idots, hipStream_t s);

}  // namespace tq
