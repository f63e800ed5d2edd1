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
  VAR_GEMV = 3,     // fp16/bf16 dot2 VALU kernel, M <= 2, activations in registers
  VAR_COUNT = 4
};

// Split-K arrival counters in the workspace: one per row group (at most 768), each on its
// own 128-byte line (a line's atomics serialize, and the row groups finish together).
constexpr int SPLIT_CTR_STRIDE = 32;   // u32 elements
constexpr int MAX_SPLIT_ROW_GROUPS = 768;

struct GemmCall {
  int fmt;            // Format
  int xt;             // 0 f32, 1 f16, 2 bf16
  const void* x;
  int M, K, N;
  const uint32_t* w;
  const uint16_t* scales;   // [N, K/G] fp16; with sbi, interleaved (scale, bias) pairs [N, K/G, 2]
  const uint16_t* biases;   // [N, K/G] fp16; null for the sign format and with sbi
  float* y;
  hipStream_t stream;
  int had_block;            // rotated format: 64, 128 or 256
  const uint32_t* signs;    // rotated format: optional sign bits [K/32]
  // grouped expert verify: the routing [M, topk] over E experts, the most rows of a job,
  // and the byte strides between consecutive experts' codes and scales (biases)
  const int32_t* route;
  int topk, E, cap;
  long long w_estride, s_estride;
  // fused argmax of every row (MFMA variants with one K slice): idx [M], and with draft
  // non-null the accepted prefix length; each workgroup's per-row keys go to amax_key
  // (FUSED_KEYS per workgroup, in the library's workspace), and launch_argmax_keys after the
  // GEMM picks the winners.
  int32_t* idx = nullptr;
  const int32_t* draft = nullptr;
  int32_t* accepted = nullptr;
  unsigned long long* amax_key = nullptr;
  // affine formats: scales holds each group's (scale, bias) pair as one word, the low half
  // the scale (one load per lane instead of one per array)
  bool sbi = false;
};

struct DeviceInfo {
  int id;             // HIP device ordinal
  int cu_count;
  int max_lds;        // bytes per workgroup
};

// Launch plan of the MFMA variants for one call.
struct MfmaPlan {
  int grid;        // workgroups = rg * ks
  int rg, ks;      // row groups, K slices (ks > 1: partials reduced by the last slice)
  int win_steps;   // K-steps per staging window (0: the call does not fit)
  int tiles_max;   // 16-row tiles per workgroup, upper bound
  int pref;        // units in flight per wave
  size_t lds;      // dynamic LDS bytes
  // One window over the whole K, one slice, and at least pref units for every wave of every
  // workgroup: a plain verify's waves store their tiles with no barrier after the loop (the
  // fused argmax and grouped jobs keep the barrier and the reduction after it).
  bool direct;
};

// Plans an MFMA call; force_ks > 0 imposes that many K slices (capped at K/1024).
// Returns false when the call cannot be staged in LDS.
bool plan_mfma(int fmt, int variant, int M, int K, int N, const DeviceInfo& dev, int force_ks,
               MfmaPlan* p);
// Plans a grouped expert verify of up to `jobs` jobs of at most M rows each (one K slice).
bool plan_mfma_grouped(int fmt, int M, int K, int N, int jobs, const DeviceInfo& dev, MfmaPlan* p);
// Plans the VALU dot2 kernel (vg_gemv): false when the call does not fit it (M > 2, K not a
// multiple of 1024 or above 16384, or the per-step partials do not fit the LDS).
bool plan_gemv(int fmt, int M, int K, int N, const DeviceInfo& dev, MfmaPlan* p);
hipError_t launch_gemv(const GemmCall& c, const MfmaPlan& p, const DeviceInfo& dev);
// Device workspace a planned call needs (partial outputs; 0 when K is not split).
size_t mfma_workspace_bytes(int M, int N, const MfmaPlan& p);

// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.
// part / counters: the call's workspace when p.ks > 1 (counters zero on entry; the
// kernel leaves them zero).
hipError_t launch_mfma(const GemmCall& c, int variant, const MfmaPlan& p, float* part,
                       uint32_t* counters, const DeviceInfo& dev);
hipError_t launch_valu(const GemmCall& c, const DeviceInfo& dev);
// Interleaves count scales and biases into (scale, bias) words: out[i] = s[i] | b[i] << 16.
hipError_t launch_pack_scale_bias(const uint16_t* s, const uint16_t* b, long long count, uint32_t* out,
                                  hipStream_t st);
hipError_t launch_hadamard(const void* x, int xt, int M, int K, int block, const uint32_t* signs, float* out,
                           hipStream_t s);
// Argmax of each row over the whole chip; with draft/accepted non-null also the greedy
// acceptance count.  pkey: argmax_chunks(N) * M parked keys, ARG_KEY_BYTES apart; counters:
// 9 zeroed words 128 bytes apart (left zeroed).
int argmax_chunks(int N);
hipError_t launch_argmax(const float* y, int M, int N, int32_t* idx, const int32_t* draft, int32_t* accepted,
                         unsigned long long* pkey, uint32_t* counters, hipStream_t s);
constexpr int ARG_KEY_BYTES = 128;   // workspace bytes per parked key (one line each)
// The fused argmax's second step: keys holds FUSED_KEYS 64-bit keys per workgroup of the GEMM
// (row m's at keys[FUSED_KEYS * g + m], zero for a row with no key) for G workgroups; one
// workgroup picks each row's largest (the lowest column among equal values), writes idx [M]
// and, with draft non-null, the accepted prefix length.
constexpr int FUSED_KEYS = 8;
hipError_t launch_argmax_keys(const unsigned long long* keys, int G, int M, int32_t* idx, const int32_t* draft,
                              int32_t* accepted, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16) from buf with loads_in_flight (1, 2, 4, 8 or
// 16) 16-byte loads per thread and wgs_per_cu (1..32) workgroups of 256 threads per CU; one
// word per workgroup to sink, which holds stream_read_blocks(dev) words.
int stream_read_blocks(const DeviceInfo& dev);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int loads_in_flight, int wgs_per_cu,
                              const DeviceInfo& dev, hipStream_t s);
// Codes of packed words as one byte per weight [N, K], decoded with the GEMM's register
// extraction for (fmt, xt) (xt F16 or BF16: the 1-bit formats decode to bf16 against bf16
// activations); 0xFF marks a half that is not an exact code.
// Static scratch of the allocation-free entry point: STATIC_SCRATCH_BYTES of device memory
// per GPU.  static_scratch returns its address on device `dev` (the current device), taken
// with hipGetSymbolAddress on the first call for that device, which also clears its first
// clear_bytes (the counter area) with a kernel on stream s.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)4 << 20;
hipError_t static_scratch(int dev, size_t clear_bytes, hipStream_t s, char** ptr);
hipError_t launch_debug_decode(int fmt, int xt, const uint32_t* w, int N, int K, uint8_t* codes,
                               hipStream_t s);

}  // namespace vg
