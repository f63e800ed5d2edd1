// vg_launch.h -- internal interface between the C-ABI layer (vg_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vg {

// Kernel variants the per-shape dispatch chooses from.  The name of each variant is the
// prefix of its kernel symbols, so a rocprofv3 trace shows which one ran.
enum Variant : int {
  VAR_MFMA_Q = 0,   // MFMA 16x16x32 f16, 16 rows = 4 row-blocks of 4 (M <= 4)
  VAR_MFMA_H = 1,   // MFMA 16x16x32 f16, 16 rows = 2 row-blocks of 8 (M <= 8)
  VAR_VALU = 2,     // plain fp32 VALU kernel (any dtype, any M; fp32 activations)
  VAR_COUNT = 3
};

struct GemmCall {
  int fmt;            // Format
  int xt;             // 0 f32, 1 f16, 2 bf16
  const void* x;
  int M, K, N;
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;  // null for the 1-bit format
  float* y;
  hipStream_t stream;
};

struct DeviceInfo {
  int id;             // HIP device ordinal
  int cu_count;
  int max_lds;        // bytes per workgroup
};

// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.
hipError_t launch_mfma(const GemmCall& c, int variant, const DeviceInfo& dev);
hipError_t launch_valu(const GemmCall& c, const DeviceInfo& dev);
hipError_t launch_hadamard(const void* x, int xt, int M, int K, float* out, hipStream_t s);
hipError_t launch_argmax(const float* y, int M, int N, int32_t* idx, hipStream_t s);
hipError_t launch_debug_unpack(int fmt, const uint32_t* w, int N, int K, uint8_t* codes,
                               hipStream_t s);

// LDS bytes the MFMA kernel needs for a call, and the K-steps per staging window it uses
// (0 if the call does not fit in `max_lds`).
size_t mfma_lds_bytes(int fmt, int variant, int M, int K, int N, int grid, int max_lds,
                      int* win_steps);

}  // namespace vg
