// vg_api.cpp -- the C ABI: argument validation, per-shape dispatch and launches.
//
// Every entry point validates its arguments on the host before touching the device, so an
// invalid call enqueues nothing and returns a status with a message (a pack declaring a
// transform that cannot be applied is refused rather than run as the plain format:
// "Ishizuki" README; failures become errors, not crashes: "Ishizuki" release notes).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/verify_gemm.h"
#include "vg_device.h"
#include "vg_launch.h"

namespace {

thread_local char g_err[512] = "";
int g_forced = -1;  // forced variant (-1: dispatch)
int g_forced_ks = 0;  // forced K slices of the MFMA variants (0: dispatch)
bool g_barrier_tail = false;  // every MFMA call sums shared tiles after a workgroup barrier
std::once_flag g_env_once;

vg_status fail(vg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

void read_env() {
  const char* v = std::getenv("VG_FORCE_VARIANT");
  if (!v || !*v) return;
  for (int i = 0; i < vg::VAR_COUNT; ++i)
    if (std::strcmp(v, vg_variant_name(i)) == 0) g_forced = i;
}

constexpr int kMaxDevices = 64;
vg::DeviceInfo g_dev[kMaxDevices];
bool g_dev_ok[kMaxDevices];
std::mutex g_dev_mu;

vg_status device_info(vg::DeviceInfo* out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices)
    return fail(VG_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ok[d]) {
    int cu = 0, lds = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, d) != hipSuccess)
      return fail(VG_ERR_HIP, "hipDeviceGetAttribute failed on device %d", d);
    g_dev[d].id = d;
    g_dev[d].cu_count = cu > 0 ? cu : 1;
    g_dev[d].max_lds = lds;
    g_dev_ok[d] = true;
  }
  *out = g_dev[d];
  return VG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vg_status check_common(const void* x, int x_dtype, int M, int K, int N) {
  if (x_dtype != VG_F32 && x_dtype != VG_F16 && x_dtype != VG_BF16)
    return fail(VG_ERR_DTYPE, "unknown activation dtype %d", x_dtype);
  if (M < 1 || M > VG_MAX_ROWS) return fail(VG_ERR_SHAPE, "M=%d outside 1..%d", M, VG_MAX_ROWS);
  if (N < 1) return fail(VG_ERR_SHAPE, "N=%d < 1", N);
  if (K < 1) return fail(VG_ERR_SHAPE, "K=%d < 1", K);
  if (!x) return fail(VG_ERR_ARG, "x is null");
  if (!aligned16(x)) return fail(VG_ERR_ALIGN, "x is not 16-byte aligned");
  return VG_OK;
}

vg_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(VG_ERR_ARG, "%s is null", name);
  if (!aligned16(p)) return fail(VG_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return VG_OK;
}

// The biases of an affine format: a separate array, or null when scales holds the
// interleaved (scale, bias) pairs.
vg_status check_biases(const void* p) {
  if (p && !aligned16(p)) return fail(VG_ERR_ALIGN, "biases is not 16-byte aligned");
  return VG_OK;
}

int kstep_of(int fmt) { (void)fmt; return 1024; }   // K per MFMA-kernel unit, both formats

// Per-shape dispatch.  fp32 activations take the exact fp32 VALU kernel.  fp16/bf16 take
// the MFMA kernels when K is a whole number of 4-group steps: mode Q up to 4 rows, mode H
// up to 8.  One row of an affine format (2-bit, or 1-bit with biases) on up to 64 MiB of
// codes takes the dot2 kernel instead, for a plain call: timed against mode Q on the
// 5120 x 17408 projections it finishes first (its set-up before the first weight load is
// shorter), while on the 151936-row output head, where that set-up no longer matters, its
// stream is slower, as it is for the sign format and the rotated format at every size
// timed.  The exception is the 1-bit affine format where mode Q finishes its tiles without
// the barrier after its loop (MfmaPlan::direct): mode Q is then ahead by 0.03-0.2 us on the
// 5120 x 17408 projection, in every one of four alternating repeats on MI355X.  A call
// that also wants the rows' argmax stays on mode Q, whose epilogue fuses the argmax: the
// dot2 kernel and the argmax kernel after it measured slower there.  Shapes the MFMA
// kernels cannot stage fall back to the VALU kernel.
constexpr double kGemvMaxCodeBytes = 64.0 * 1024 * 1024;
int plan(int fmt, int xt, int M, int N, int K, const vg::DeviceInfo& dev, bool argmax = false) {
  if (xt == VG_F32) return vg::VAR_VALU;
  if (K % kstep_of(fmt) != 0) return vg::VAR_VALU;
  if (!argmax && M == 1 && (fmt == vg::AFFINE2 || fmt == vg::AFFINE1) &&
      (double)N * K / (fmt == vg::AFFINE2 ? 4.0 : 8.0) <= kGemvMaxCodeBytes) {
    vg::MfmaPlan q;
    const bool q_direct = fmt == vg::AFFINE1 && vg::plan_mfma(fmt, vg::VAR_MFMA_Q, M, K, N, dev, g_forced_ks, &q) &&
                          q.direct;
    vg::MfmaPlan g;
    if (!q_direct && vg::plan_gemv(fmt, M, K, N, dev, &g)) return vg::VAR_GEMV;
  }
  const int var = M <= 4 ? vg::VAR_MFMA_Q : vg::VAR_MFMA_H;
  vg::MfmaPlan p;
  return vg::plan_mfma(fmt, var, M, K, N, dev, g_forced_ks, &p) ? var : vg::VAR_VALU;
}

bool variant_supports(int var, int fmt, int xt, int M, int N, int K, const vg::DeviceInfo& dev) {
  if (var == vg::VAR_VALU) return true;
  if (xt == VG_F32 || K % kstep_of(fmt) != 0) return false;
  if (var == vg::VAR_GEMV) {
    vg::MfmaPlan p;
    return vg::plan_gemv(fmt, M, K, N, dev, &p);
  }
  if (var == vg::VAR_MFMA_Q && M > 4) return false;
  vg::MfmaPlan p;
  return vg::plan_mfma(fmt, var, M, K, N, dev, g_forced_ks, &p);
}

// Workspaces of the calls that split K across workgroups and of the argmax calls, one per
// (device, stream): the partial outputs, the arrival counters and the argmax keys.  Created
// on the first such call on a stream and replaced by a larger one when a call needs more.
// A replaced buffer is never freed while the process runs (it goes on a retired list):
// work already enqueued, or a graph captured earlier, may still use it.  Creating or
// growing needs hipMalloc and a clear of the counters, so a call under stream capture
// that would need either is refused (VG_ERR_UNSUPPORTED) before anything is enqueued.
// The kernels leave counters and keys zero, so consecutive calls on one stream share them;
// calls on different streams never share a workspace.
struct Workspace {
  int dev;
  hipStream_t stream;
  char* ptr;
  size_t bytes;
  std::vector<void*> retired;
};
std::mutex g_ws_mu;
std::vector<Workspace> g_ws;
// Counter area (zeroed at allocation, left zero by every call), u32 indices, each counter on
// its own 128-byte line:
//   [0, 24576)       split-K arrival counters, row group r at r * 32 (r < 768)
//   [24576, 24864)   the argmax kernel's nine counters (rows 0..7, finished rows)
// The fused argmax needs no counter: its per-workgroup keys sit in the partial area.
constexpr int kArgmaxCounterBase = vg::MAX_SPLIT_ROW_GROUPS * vg::SPLIT_CTR_STRIDE;
constexpr size_t kCounterBytes = 116736;
static_assert((kArgmaxCounterBase + 32 * (VG_MAX_ROWS + 1)) * 4 <= (int)kCounterBytes, "counter area too small");

// Whether work enqueued on `stream` now would be captured into a graph.
bool capturing(hipStream_t stream, bool* cap) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
  *cap = st != hipStreamCaptureStatusNone;
  return true;
}

vg_status workspace(int dev, hipStream_t stream, size_t part_bytes, float** part, uint32_t** counters) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  for (auto& e : g_ws)
    if (e.dev == dev && e.stream == stream) w = &e;
  const size_t need = kCounterBytes + part_bytes;
  if (!w || w->bytes < need) {
    bool cap = false;
    if (!capturing(stream, &cap)) return fail(VG_ERR_HIP, "querying the stream's capture status failed");
    if (cap)
      return fail(VG_ERR_UNSUPPORTED,
                  "this call needs a %zu-byte workspace on the capturing stream, which has %s: make one "
                  "eager call of this size on the stream before capturing it",
                  need, w ? "a smaller one" : "none");
    const size_t bytes = need + need / 2;
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return fail(VG_ERR_HIP, "workspace allocation of %zu bytes failed", bytes);
    if (hipMemsetAsync(p, 0, kCounterBytes, stream) != hipSuccess) {
      (void)hipFree(p);
      return fail(VG_ERR_HIP, "clearing the workspace counters failed");
    }
    if (!w) {
      g_ws.push_back(Workspace{dev, stream, nullptr, 0, {}});
      w = &g_ws.back();
    }
    if (w->ptr) w->retired.push_back(w->ptr);   // earlier calls on the stream may still use it
    w->ptr = static_cast<char*>(p);
    w->bytes = bytes;
  }
  *counters = reinterpret_cast<uint32_t*>(w->ptr);
  *part = reinterpret_cast<float*>(w->ptr + kCounterBytes);
  return VG_OK;
}

// Frees the current device's workspace of `stream` (after synchronizing the stream).
vg_status release_workspace(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VG_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (size_t k = 0; k < g_ws.size(); ++k) {
    Workspace& w = g_ws[k];
    if (w.dev != dev || w.stream != stream) continue;
    bool cap = false;
    if (!capturing(stream, &cap)) return fail(VG_ERR_HIP, "querying the stream's capture status failed");
    if (cap) return fail(VG_ERR_UNSUPPORTED, "the stream is capturing a graph");
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(VG_ERR_HIP, "synchronizing the stream failed");
    bool ok = hipFree(w.ptr) == hipSuccess;
    for (void* r : w.retired) ok = hipFree(r) == hipSuccess && ok;
    g_ws.erase(g_ws.begin() + (long)k);
    if (!ok) return fail(VG_ERR_HIP, "freeing the workspace failed");
    return VG_OK;
  }
  return VG_OK;
}

// Where a call's workspace comes from: the stream's workspace above (created on first
// use), or a fixed region given by the caller of run_gemm (the static scratch of
// verify_gemm_argmax_noalloc), which is refused when the call needs more than it holds.
struct Fixed {
  size_t bytes;   // the static scratch's size; its address is looked up on first use
};

vg_status get_workspace(const Fixed* fixed, int dev, hipStream_t stream, size_t part_bytes, float** part,
                        uint32_t** counters) {
  if (!fixed) return workspace(dev, stream, part_bytes, part, counters);
  if (kCounterBytes + part_bytes > fixed->bytes)
    return fail(VG_ERR_UNSUPPORTED, "the call needs %zu bytes of scratch, above the static maximum of %zu",
                kCounterBytes + part_bytes, fixed->bytes);
  char* base = nullptr;
  const hipError_t e = vg::static_scratch(dev, kCounterBytes, stream, &base);
  if (e != hipSuccess) return fail(VG_ERR_HIP, "static scratch set-up failed: %s", hipGetErrorString(e));
  *counters = reinterpret_cast<uint32_t*>(base);
  *part = reinterpret_cast<float*>(base + kCounterBytes);
  return VG_OK;
}

// The argmax kernel's parked keys (bytes in the workspace's partial area).
size_t argmax_key_bytes(int M, int N) { return (size_t)vg::argmax_chunks(N) * M * vg::ARG_KEY_BYTES; }

vg_status launch_argmax_ws(const float* y, int M, int N, int32_t* idx, const int32_t* draft, int32_t* accepted,
                           float* part, uint32_t* counters, hipStream_t st) {
  const hipError_t e = vg::launch_argmax(y, M, N, idx, draft, accepted, reinterpret_cast<unsigned long long*>(part),
                                         counters + kArgmaxCounterBase, st);
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return VG_OK;
}

// The verify GEMM; with idx non-null also the argmax of every row (and the accepted prefix
// when draft is non-null): fused into the GEMM's epilogue when the plan runs the MFMA
// kernels with one K slice, else the argmax kernel after it (same results either way).
// Everything the call needs (split-K partials, counters, argmax keys) is acquired before
// the first launch, so a refused call enqueues nothing.
vg_status run_gemm(int fmt, const void* x, int x_dtype, int M, int K, const uint32_t* w,
                   const uint16_t* scales, const uint16_t* biases, int N, float* y, void* stream,
                   int had_block = 128, const uint32_t* signs = nullptr, int32_t* idx = nullptr,
                   const int32_t* draft = nullptr, int32_t* accepted = nullptr, const Fixed* fixed = nullptr) {
  std::call_once(g_env_once, read_env);
  vg::DeviceInfo dev;
  if (vg_status s = device_info(&dev)) return s;
  int var = plan(fmt, x_dtype, M, N, K, dev, idx != nullptr);
  if (g_forced >= 0) {
    if (!variant_supports(g_forced, fmt, x_dtype, M, N, K, dev))
      return fail(VG_ERR_UNSUPPORTED, "forced variant %s cannot run format %d dtype %d M=%d K=%d",
                  vg_variant_name(g_forced), fmt, x_dtype, M, K);
    var = g_forced;
  }
  vg::GemmCall c{fmt, x_dtype, x, M, K, N, w, scales, biases, y, static_cast<hipStream_t>(stream),
                 had_block, signs};
  c.sbi = fmt != vg::SIGN1 && biases == nullptr;
  vg::MfmaPlan p{};
  const bool mfma = var == vg::VAR_MFMA_Q || var == vg::VAR_MFMA_H;
  if (mfma) {
    if (!vg::plan_mfma(fmt, var, M, K, N, dev, g_forced_ks, &p))
      return fail(VG_ERR_UNSUPPORTED, "M=%d K=%d does not fit the MFMA staging", M, K);
    if (g_barrier_tail) p.direct = false;
    if (p.ks > 1 && p.rg > vg::MAX_SPLIT_ROW_GROUPS) return fail(VG_ERR_UNSUPPORTED, "too many row groups");
  } else if (var == vg::VAR_GEMV) {
    if (!vg::plan_gemv(fmt, M, K, N, dev, &p))
      return fail(VG_ERR_UNSUPPORTED, "M=%d K=%d does not fit the dot2 kernel's staging", M, K);
  }
  const bool split = mfma && p.ks > 1;
  const bool fused = idx && mfma && !split;
  const bool argmax_after = idx && !fused;
  float* part = nullptr;
  uint32_t* counters = nullptr;
  if (split || idx) {
    size_t part_bytes = split ? vg::mfma_workspace_bytes(M, N, p) : 0;
    if (argmax_after && argmax_key_bytes(M, N) > part_bytes) part_bytes = argmax_key_bytes(M, N);
    // the fused argmax: FUSED_KEYS 64-bit keys per workgroup
    if (fused && (size_t)p.grid * vg::FUSED_KEYS * 8 > part_bytes) part_bytes = (size_t)p.grid * vg::FUSED_KEYS * 8;
    if (vg_status s = get_workspace(fixed, dev.id, c.stream, part_bytes, &part, &counters)) return s;
  }
  hipError_t e;
  if (var == vg::VAR_VALU) {
    e = vg::launch_valu(c, dev);
  } else if (var == vg::VAR_GEMV) {
    e = vg::launch_gemv(c, p, dev);
  } else if (fused) {
    // each workgroup stores its rows' largest keys, and one workgroup after the GEMM picks
    // the winners: stream order makes the keys visible, where a count of arriving
    // workgroups inside the GEMM would add three dependent trips past the L2 to its end
    c.idx = idx;
    c.draft = draft;
    c.accepted = accepted;
    c.amax_key = reinterpret_cast<unsigned long long*>(part);
    e = vg::launch_mfma(c, var, p, nullptr, nullptr, dev);
    if (e == hipSuccess) e = vg::launch_argmax_keys(c.amax_key, p.grid, M, idx, draft, accepted, c.stream);
  } else {
    e = vg::launch_mfma(c, var, p, split ? part : nullptr, split ? counters : nullptr, dev);
  }
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  if (argmax_after)
    if (vg_status s = launch_argmax_ws(y, M, N, idx, draft, accepted, part, counters, c.stream)) return s;
  g_err[0] = '\0';
  return VG_OK;
}

// Grouped expert verify: one MFMA launch whose workgroups each group the routing by expert
// and take one row group of one job.  Mode Q (jobs of up to 4 rows) when the call has up to 4 rows, else mode H (up to 8);
// the plan depends only on (format, dtype, M, topk, E, K, N), so a row's result does not
// depend on which other rows are routed with it.
vg_status run_experts(int fmt, const void* x, int x_dtype, int M, int K, int E, int topk, const int32_t* route,
                      const uint32_t* w, const uint16_t* scales, const uint16_t* biases, int N, float* y,
                      void* stream) {
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  if (E < 1) return fail(VG_ERR_SHAPE, "E=%d < 1", E);
  if (topk < 1 || topk > VG_MAX_ROWS) return fail(VG_ERR_SHAPE, "topk=%d outside 1..%d", topk, VG_MAX_ROWS);
  if (x_dtype == VG_F32)
    return fail(VG_ERR_UNSUPPORTED, "grouped expert verify takes fp16 or bf16 activations");
  if (K % kstep_of(fmt) != 0) return fail(VG_ERR_UNSUPPORTED, "grouped expert verify needs K a multiple of 1024 (K=%d)", K);
  if (!route) return fail(VG_ERR_ARG, "route is null");
  if (reinterpret_cast<uintptr_t>(route) & 3u) return fail(VG_ERR_ALIGN, "route is not 4-byte aligned");
  if (vg_status s = check_ptr(w, "w")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (fmt != vg::SIGN1)
    if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  std::call_once(g_env_once, read_env);
  vg::DeviceInfo dev;
  if (vg_status s = device_info(&dev)) return s;
  const int var = M <= 4 ? vg::VAR_MFMA_Q : vg::VAR_MFMA_H;
  const int cap = M <= 4 ? 4 : 8;
  const int n = M * topk;
  const int rows_max = n < cap ? n : cap;   // rows of one job
  // most jobs a routing can make: each holds at least one entry, and the experts' jobs
  // number sum ceil(count / cap) <= (experts used) + n / cap
  const long long jobs_e = (long long)E + n / cap;
  const int jobs = jobs_e < n ? (int)jobs_e : n;
  vg::MfmaPlan p;
  if (!vg::plan_mfma_grouped(fmt, rows_max, K, N, jobs, dev, &p))
    return fail(VG_ERR_UNSUPPORTED, "M=%d K=%d does not fit the MFMA staging", M, K);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool two_bit = fmt == vg::AFFINE2 || fmt == vg::HAD2;
  const long long words = (long long)N * (K / (two_bit ? 16 : 32));
  const long long groups = (long long)N * (K / (two_bit ? 64 : 128));
  const bool sbi = fmt != vg::SIGN1 && biases == nullptr;
  vg::GemmCall c{fmt, x_dtype, x, M, K, N, w, scales, sbi ? nullptr : biases, y, st, 128, nullptr,
                 route, topk, E, cap, words * 4, groups * (sbi ? 4 : 2)};
  c.sbi = sbi;
  const hipError_t e = vg::launch_mfma(c, var, p, nullptr, nullptr, dev);
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return VG_OK;
}


vg_status run_argmax(const float* y, int M, int N, int32_t* idx, const int32_t* draft, int32_t* accepted,
                     void* stream) {
  if (M < 1 || M > VG_MAX_ROWS) return fail(VG_ERR_SHAPE, "M=%d outside 1..%d", M, VG_MAX_ROWS);
  if (N < 1) return fail(VG_ERR_SHAPE, "N=%d < 1", N);
  if (!y) return fail(VG_ERR_ARG, "y is null");
  if (reinterpret_cast<uintptr_t>(y) & 3u) return fail(VG_ERR_ALIGN, "y is not 4-byte aligned");
  if (!idx) return fail(VG_ERR_ARG, "idx is null");
  if ((draft == nullptr) != (accepted == nullptr)) return fail(VG_ERR_ARG, "draft and accepted go together");
  vg::DeviceInfo dev;
  if (vg_status s = device_info(&dev)) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = nullptr;
  uint32_t* counters = nullptr;
  if (vg_status s = workspace(dev.id, st, argmax_key_bytes(M, N), &part, &counters)) return s;
  if (vg_status s = launch_argmax_ws(y, M, N, idx, draft, accepted, part, counters, st)) return s;
  g_err[0] = '\0';
  return VG_OK;
}

}  // namespace

extern "C" {

vg_status verify_gemm_sign1(const void* x, int x_dtype, int M, int K, const uint32_t* wbits,
                            const uint16_t* scales, int N, float* y, void* stream) {
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  if (K % 128 != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of 128 (1-bit group)", K);
  if (vg_status s = check_ptr(wbits, "wbits")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  return run_gemm(vg::SIGN1, x, x_dtype, M, K, wbits, scales, nullptr, N, y, stream);
}

vg_status verify_gemm_affine1(const void* x, int x_dtype, int M, int K, const uint32_t* wbits,
                              const uint16_t* scales, const uint16_t* biases, int N, float* y,
                              void* stream) {
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  if (K % 128 != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of 128 (1-bit affine group)", K);
  if (vg_status s = check_ptr(wbits, "wbits")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  return run_gemm(vg::AFFINE1, x, x_dtype, M, K, wbits, scales, biases, N, y, stream);
}

vg_status verify_gemm_affine2(const void* x, int x_dtype, int M, int K, const uint32_t* wq,
                              const uint16_t* scales, const uint16_t* biases, int N, float* y,
                              void* stream) {
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  if (K % 64 != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of 64 (2-bit group)", K);
  if (vg_status s = check_ptr(wq, "wq")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  return run_gemm(vg::AFFINE2, x, x_dtype, M, K, wq, scales, biases, N, y, stream);
}

vg_status verify_gemm_had2_signed(const void* x, int x_dtype, int M, int K, const uint32_t* wq,
                                  const uint16_t* scales, const uint16_t* biases, int N, int had_block,
                                  const uint32_t* signs, float* y, void* stream) {
  if (had_block != 64 && had_block != 128 && had_block != 256)
    return fail(VG_ERR_UNSUPPORTED, "Hadamard block %d is not supported (64, 128 or 256)", had_block);
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  if (K % 128 != 0 || K % had_block != 0)
    return fail(VG_ERR_SHAPE, "K=%d is not a multiple of 128 and of the Hadamard block %d", K, had_block);
  if (vg_status s = check_ptr(wq, "wq")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  if (signs && (reinterpret_cast<uintptr_t>(signs) & 3u)) return fail(VG_ERR_ALIGN, "signs is not 4-byte aligned");
  return run_gemm(vg::HAD2, x, x_dtype, M, K, wq, scales, biases, N, y, stream, had_block, signs);
}

vg_status verify_gemm_had2(const void* x, int x_dtype, int M, int K, const uint32_t* wq,
                           const uint16_t* scales, const uint16_t* biases, int N, int had_block,
                           float* y, void* stream) {
  return verify_gemm_had2_signed(x, x_dtype, M, K, wq, scales, biases, N, had_block, nullptr, y, stream);
}

vg_status hadamard_rotate_signed(const void* x, int x_dtype, int M, int K, int block, const uint32_t* signs,
                                 float* x_out, void* stream) {
  if (block != 64 && block != 128 && block != 256)
    return fail(VG_ERR_UNSUPPORTED, "Hadamard block %d is not supported (64, 128 or 256)", block);
  if (vg_status s = check_common(x, x_dtype, M, K, 1)) return s;
  if (K % block != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of the Hadamard block %d", K, block);
  if (vg_status s = check_ptr(x_out, "x_out")) return s;
  if (signs && (reinterpret_cast<uintptr_t>(signs) & 3u)) return fail(VG_ERR_ALIGN, "signs is not 4-byte aligned");
  const hipError_t e = vg::launch_hadamard(x, x_dtype, M, K, block, signs, x_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return VG_OK;
}

vg_status hadamard_rotate(const void* x, int x_dtype, int M, int K, int block, float* x_out,
                          void* stream) {
  return hadamard_rotate_signed(x, x_dtype, M, K, block, nullptr, x_out, stream);
}

vg_status verify_gemm_argmax(int format, const void* x, int x_dtype, int M, int K, const uint32_t* w,
                             const uint16_t* scales, const uint16_t* biases, int N, float* y, int32_t* idx,
                             const int32_t* draft, int32_t* accepted, void* stream) {
  if (format != vg::SIGN1 && format != vg::AFFINE2 && format != vg::HAD2 && format != vg::AFFINE1)
    return fail(VG_ERR_ARG, "unknown format %d", format);
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  const int G = vg::fmt_one_bit(format) || format == vg::HAD2 ? 128 : 64;
  if (K % G != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of %d", K, G);
  if (vg_status s = check_ptr(w, "w")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (format != vg::SIGN1)
    if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  if (!idx) return fail(VG_ERR_ARG, "idx is null");
  if (reinterpret_cast<uintptr_t>(idx) & 3u) return fail(VG_ERR_ALIGN, "idx is not 4-byte aligned");
  if ((draft == nullptr) != (accepted == nullptr)) return fail(VG_ERR_ARG, "draft and accepted go together");
  return run_gemm(format, x, x_dtype, M, K, w, scales, format == vg::SIGN1 ? nullptr : biases, N, y, stream, 128,
                  nullptr, idx, draft, accepted);
}

vg_status verify_gemm_argmax_noalloc(int format, const void* x, int x_dtype, int M, int K, const uint32_t* w,
                                     const uint16_t* scales, const uint16_t* biases, int N, float* y,
                                     int32_t* idx, const int32_t* draft, int32_t* accepted, void* stream) {
  if (format != vg::SIGN1 && format != vg::AFFINE2 && format != vg::HAD2 && format != vg::AFFINE1)
    return fail(VG_ERR_ARG, "unknown format %d", format);
  if (vg_status s = check_common(x, x_dtype, M, K, N)) return s;
  const int G = vg::fmt_one_bit(format) || format == vg::HAD2 ? 128 : 64;
  if (K % G != 0) return fail(VG_ERR_SHAPE, "K=%d is not a multiple of %d", K, G);
  if (vg_status s = check_ptr(w, "w")) return s;
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (format != vg::SIGN1)
    if (vg_status s = check_biases(biases)) return s;
  if (vg_status s = check_ptr(y, "y")) return s;
  if (idx && (reinterpret_cast<uintptr_t>(idx) & 3u)) return fail(VG_ERR_ALIGN, "idx is not 4-byte aligned");
  if ((draft == nullptr) != (accepted == nullptr)) return fail(VG_ERR_ARG, "draft and accepted go together");
  if (draft && !idx) return fail(VG_ERR_ARG, "draft needs idx");
  const Fixed fixed{vg::STATIC_SCRATCH_BYTES};
  return run_gemm(format, x, x_dtype, M, K, w, scales, format == vg::SIGN1 ? nullptr : biases, N, y, stream, 128,
                  nullptr, idx, draft, accepted, &fixed);
}

vg_status verify_argmax_rows(const float* y, int M, int N, int32_t* idx, void* stream) {
  return run_argmax(y, M, N, idx, nullptr, nullptr, stream);
}

vg_status verify_accept_greedy(const float* y, int M, int N, const int32_t* draft, int32_t* idx,
                               int32_t* accepted, void* stream) {
  if (!draft || !accepted) return fail(VG_ERR_ARG, "draft or accepted is null");
  return run_argmax(y, M, N, idx, draft, accepted, stream);
}

vg_status verify_gemm_experts(int format, const void* x, int x_dtype, int M, int K, int E, int topk,
                              const int32_t* route, const uint32_t* w, const uint16_t* scales,
                              const uint16_t* biases, int N, float* y, void* stream) {
  if (format < VG_FMT_SIGN1 || format > VG_FMT_AFFINE1) return fail(VG_ERR_ARG, "unknown format %d", format);
  return run_experts(format, x, x_dtype, M, K, E, topk, route, w, scales, biases, N, y, stream);
}

vg_status vg_pack_scale_bias(const uint16_t* scales, const uint16_t* biases, long long count, uint16_t* out,
                             void* stream) {
  if (count < 0) return fail(VG_ERR_SHAPE, "count=%lld < 0", count);
  if (vg_status s = check_ptr(scales, "scales")) return s;
  if (vg_status s = check_ptr(biases, "biases")) return s;
  if (vg_status s = check_ptr(out, "out")) return s;
  const auto overlaps = [count](const void* a, long long abytes, const void* b, long long bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return count > 0 && a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
  };
  if (overlaps(out, 4 * count, scales, 2 * count) || overlaps(out, 4 * count, biases, 2 * count))
    return fail(VG_ERR_ARG, "out overlaps scales or biases");
  const hipError_t e = vg::launch_pack_scale_bias(scales, biases, count, reinterpret_cast<uint32_t*>(out),
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return VG_OK;
}

const char* vg_last_error(void) { return g_err; }

vg_status vg_release_stream_workspace(void* stream) {
  const vg_status s = release_workspace(static_cast<hipStream_t>(stream));
  if (s == VG_OK) g_err[0] = '\0';
  return s;
}

int vg_plan_variant(int format, int x_dtype, int M, int N, int K) {
  if (format < 0 || format > 3) return -1;
  if (x_dtype < 0 || x_dtype > 2 || M < 1 || M > VG_MAX_ROWS || N < 1 || K < 1) return -1;
  if (K % (format == vg::AFFINE2 ? 64 : 128) != 0) return -1;
  std::call_once(g_env_once, read_env);
  vg::DeviceInfo dev;
  if (device_info(&dev) != VG_OK) return -1;
  if (g_forced >= 0) return variant_supports(g_forced, format, x_dtype, M, N, K, dev) ? g_forced : -1;
  return plan(format, x_dtype, M, N, K, dev);
}

const char* vg_variant_name(int variant) {
  switch (variant) {
    case vg::VAR_MFMA_Q: return "vg_mfma_q";
    case vg::VAR_MFMA_H: return "vg_mfma_h";
    case vg::VAR_VALU: return "vg_valu";
    case vg::VAR_GEMV: return "vg_gemv";
    default: return "";
  }
}

vg_status vg_force_variant(int variant) {
  std::call_once(g_env_once, read_env);
  if (variant < -1 || variant >= vg::VAR_COUNT) return fail(VG_ERR_ARG, "unknown variant %d", variant);
  g_forced = variant;
  return VG_OK;
}

int vg_variant_count(void) { return vg::VAR_COUNT; }

vg_status vg_force_ksplit(int ksplit) {
  if (ksplit < 0 || ksplit > 64) return fail(VG_ERR_ARG, "K slices %d outside 0..64", ksplit);
  g_forced_ks = ksplit;
  return VG_OK;
}

int vg_plan_ksplit(int format, int x_dtype, int M, int N, int K) {
  const int var = vg_plan_variant(format, x_dtype, M, N, K);
  if (var < 0) return -1;
  if (var == vg::VAR_VALU || var == vg::VAR_GEMV) return 1;
  vg::DeviceInfo dev;
  if (device_info(&dev) != VG_OK) return -1;
  vg::MfmaPlan p;
  return vg::plan_mfma(format, var, M, K, N, dev, g_forced_ks, &p) ? p.ks : -1;
}

vg_status vg_force_barrier_tail(int on) {
  if (on != 0 && on != 1) return fail(VG_ERR_ARG, "barrier tail flag %d is not 0 or 1", on);
  g_barrier_tail = on == 1;
  return VG_OK;
}

int vg_plan_direct(int format, int x_dtype, int M, int N, int K) {
  const int var = vg_plan_variant(format, x_dtype, M, N, K);
  if (var < 0) return -1;
  if (var == vg::VAR_VALU || var == vg::VAR_GEMV) return 0;
  vg::DeviceInfo dev;
  if (device_info(&dev) != VG_OK) return -1;
  vg::MfmaPlan p;
  if (!vg::plan_mfma(format, var, M, K, N, dev, g_forced_ks, &p)) return -1;
  return p.direct && !g_barrier_tail ? 1 : 0;
}

int vg_stream_read_blocks(void) {
  vg::DeviceInfo dev;
  if (device_info(&dev) != VG_OK) return -1;
  return vg::stream_read_blocks(dev);
}

vg_status vg_stream_read_config(const void* buf, size_t bytes, uint32_t* sink, int loads_in_flight, int wgs_per_cu,
                                void* stream) {
  if (vg_status s = check_ptr(buf, "buf")) return s;
  if (bytes == 0 || bytes % 16 != 0) return fail(VG_ERR_SHAPE, "bytes=%zu is not a positive multiple of 16", bytes);
  if (!sink) return fail(VG_ERR_ARG, "sink is null");
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return fail(VG_ERR_ALIGN, "sink is not 4-byte aligned");
  if (loads_in_flight != 1 && loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8 &&
      loads_in_flight != 16)
    return fail(VG_ERR_ARG, "loads in flight %d is not 1, 2, 4, 8 or 16", loads_in_flight);
  if (wgs_per_cu < 1 || wgs_per_cu > 32) return fail(VG_ERR_ARG, "workgroups per CU %d outside 1..32", wgs_per_cu);
  vg::DeviceInfo dev;
  if (vg_status s = device_info(&dev)) return s;
  const hipError_t e = vg::launch_stream_read(buf, bytes, sink, loads_in_flight, wgs_per_cu, dev,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return VG_OK;
}

vg_status vg_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  return vg_stream_read_config(buf, bytes, sink, 4, 8, stream);
}

vg_status vg_debug_unpack(int format, int x_dtype, const uint32_t* w, int N, int K, uint8_t* codes,
                          void* stream) {
  if (format < VG_FMT_SIGN1 || format > VG_FMT_AFFINE1) return fail(VG_ERR_ARG, "unknown format %d", format);
  if (x_dtype == VG_F32)
    return fail(VG_ERR_UNSUPPORTED, "fp32 activations take the VALU kernel, which has no register decode");
  if (x_dtype != VG_F16 && x_dtype != VG_BF16) return fail(VG_ERR_DTYPE, "unknown activation dtype %d", x_dtype);
  const int wk = vg::fmt_one_bit(format) ? 32 : 16;
  if (N < 1 || K < wk || K % wk != 0) return fail(VG_ERR_SHAPE, "bad shape N=%d K=%d", N, K);
  if ((long long)N * (K / wk) > (1ll << 38)) return fail(VG_ERR_SHAPE, "N=%d K=%d is too large", N, K);
  if (vg_status s = check_ptr(w, "w")) return s;
  if (!codes) return fail(VG_ERR_ARG, "codes is null");
  const hipError_t e = vg::launch_debug_decode(format, x_dtype, w, N, K, codes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return VG_OK;
}

vg_status vg_debug_unpack_sign1(const uint32_t* wbits, int N, int K, uint8_t* codes, void* stream) {
  return vg_debug_unpack(VG_FMT_SIGN1, VG_F16, wbits, N, K, codes, stream);
}

vg_status vg_debug_unpack_affine2(const uint32_t* wq, int N, int K, uint8_t* codes, void* stream) {
  return vg_debug_unpack(VG_FMT_AFFINE2, VG_F16, wq, N, K, codes, stream);
}

}  // extern "C"
