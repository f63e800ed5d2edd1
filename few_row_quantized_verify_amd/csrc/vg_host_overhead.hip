// vg_host_overhead.hip -- host time of one verify call through the C ABI (argument checks,
// plan, kernel launch), measured natively beside a bare kernel launch.  While each block of
// calls is enqueued, the GPU is held busy by a streaming read of 1 GiB, so every call only
// enqueues and the host clock sees the library's own cost.  Shape: the 2-bit affine
// 5120 x 17408 projection with interleaved scale-and-bias pairs, every row count 1..8.
// Prints one JSON object.  Usage: vg_host_overhead [calls per block] [blocks]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "verify_gemm.h"

__global__ void vg_empty_kernel() {}

// Kernels taking an argument block of 64 bytes and of the verify kernels' 304 bytes, to
// separate the cost of the launch with its arguments from the library's own.
template <int BYTES>
struct Args {
  unsigned char b[BYTES];
};
template <int BYTES>
__global__ void vg_args_kernel(Args<BYTES> a) {
  if (a.b[0] == 1 && threadIdx.x == 0) a.b[1] = 2;
}

#define CK(x)                                                                               \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
      return 2;                                                                             \
    }                                                                                       \
  } while (0)
#define VG(x)                                                                               \
  do {                                                                                      \
    vg_status s_ = (x);                                                                     \
    if (s_ != VG_OK) {                                                                      \
      std::fprintf(stderr, "vg error %d (%s) at line %d\n", (int)s_, vg_last_error(), __LINE__); \
      return 3;                                                                             \
    }                                                                                       \
  } while (0)

static double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

int main(int argc, char** argv) {
  const int calls = argc > 1 ? std::atoi(argv[1]) : 200;
  const int blocks = argc > 2 ? std::atoi(argv[2]) : 7;
  if (calls < 1 || calls > 1000 || blocks < 1 || blocks > 100) {
    std::fprintf(stderr, "calls per block in 1..1000, blocks in 1..100\n");
    return 1;
  }
  const int K = 5120, N = 17408, MMAX = 8;
  const size_t hold_bytes = (size_t)1 << 30;
  void *x, *w, *sb, *y, *hold, *sink;
  CK(hipMalloc(&x, (size_t)MMAX * K * 2));
  CK(hipMalloc(&w, (size_t)N * K / 4));
  CK(hipMalloc(&sb, (size_t)N * (K / 64) * 4));
  CK(hipMalloc(&y, (size_t)MMAX * N * 4));
  CK(hipMalloc(&hold, hold_bytes));
  CK(hipMalloc(&sink, (size_t)vg_stream_read_blocks() * 4));
  // zero codes, scales, biases and activations are valid inputs; only the time is measured
  CK(hipMemset(x, 0, (size_t)MMAX * K * 2));
  CK(hipMemset(w, 0, (size_t)N * K / 4));
  CK(hipMemset(sb, 0, (size_t)N * (K / 64) * 4));
  CK(hipMemset(hold, 0, hold_bytes));
  hipStream_t st;
  CK(hipStreamCreate(&st));
  auto call = [&](int M) {
    return verify_gemm_affine2(x, VG_F16, M, K, static_cast<const uint32_t*>(w), static_cast<const uint16_t*>(sb),
                               nullptr, N, static_cast<float*>(y), st);
  };
  for (int M = 1; M <= MMAX; ++M)
    for (int i = 0; i < 50; ++i) VG(call(M));
  for (int i = 0; i < 50; ++i) hipLaunchKernelGGL(vg_empty_kernel, dim3(1), dim3(64), 0, st);
  CK(hipGetLastError());
  CK(hipStreamSynchronize(st));

  using clk = std::chrono::steady_clock;
  // host-only reference points: the plan queries (device lookup and per-shape plan, no launch)
  std::vector<double> plan_us;
  for (int b = 0; b < blocks; ++b) {
    const auto t0 = clk::now();
    int acc = 0;
    for (int i = 0; i < calls; ++i) acc += vg_plan_variant(VG_FMT_AFFINE2, VG_F16, 1 + i % MMAX, N, K);
    const auto t1 = clk::now();
    if (acc < 0) return 4;
    plan_us.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count() / calls);
  }
  Args<304> big{};
  Args<64> small{};
  for (int i = 0; i < 50; ++i) {
    hipLaunchKernelGGL(vg_args_kernel<304>, dim3(1), dim3(64), 0, st, big);
    hipLaunchKernelGGL(vg_args_kernel<64>, dim3(1), dim3(64), 0, st, small);
  }
  CK(hipStreamSynchronize(st));
  std::vector<double> per_m[MMAX + 1], empty, bigv, smallv;
  for (int b = 0; b < blocks; ++b) {
    for (int M = -2; M <= MMAX; ++M) {   // bare launches: -2 with 64 bytes of arguments, -1 with 304, 0 with none
      VG(vg_stream_read(hold, hold_bytes, static_cast<uint32_t*>(sink), st));
      const auto t0 = clk::now();
      if (M == 0) {
        for (int i = 0; i < calls; ++i) hipLaunchKernelGGL(vg_empty_kernel, dim3(1), dim3(64), 0, st);
      } else if (M == -1) {
        for (int i = 0; i < calls; ++i) hipLaunchKernelGGL(vg_args_kernel<304>, dim3(1), dim3(64), 0, st, big);
      } else if (M == -2) {
        for (int i = 0; i < calls; ++i) hipLaunchKernelGGL(vg_args_kernel<64>, dim3(1), dim3(64), 0, st, small);
      } else {
        for (int i = 0; i < calls; ++i) VG(call(M));
      }
      const auto t1 = clk::now();
      CK(hipGetLastError());
      CK(hipStreamSynchronize(st));
      const double us = std::chrono::duration<double, std::micro>(t1 - t0).count() / calls;
      (M == 0 ? empty : (M == -1 ? bigv : (M == -2 ? smallv : per_m[M]))).push_back(us);
    }
  }
  std::printf("{\"host_overhead\": {\"shape\": \"affine2 K=%d N=%d, interleaved scales and biases\", "
              "\"calls_per_block\": %d, \"blocks\": %d, \"empty_kernel_launch_us\": %.3f, "
              "\"launch_with_64_byte_args_us\": %.3f, \"launch_with_304_byte_args_us\": %.3f, "
              "\"plan_query_us\": %.3f, \"verify_call_us\": {",
              K, N, calls, blocks, median(empty), median(smallv), median(bigv), median(plan_us));
  for (int M = 1; M <= MMAX; ++M) std::printf("%s\"%d\": %.3f", M > 1 ? ", " : "", M, median(per_m[M]));
  std::printf("}, \"variant\": {");
  for (int M = 1; M <= MMAX; ++M)
    std::printf("%s\"%d\": \"%s\"", M > 1 ? ", " : "", M, vg_variant_name(vg_plan_variant(VG_FMT_AFFINE2, VG_F16, M, N, K)));
  std::printf("}}}\n");
  CK(hipStreamDestroy(st));
  CK(hipFree(x));
  CK(hipFree(w));
  CK(hipFree(sb));
  CK(hipFree(y));
  CK(hipFree(hold));
  CK(hipFree(sink));
  return 0;
}
