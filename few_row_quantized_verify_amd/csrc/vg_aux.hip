// vg_aux.hip -- the VALU verify kernel (fp32 activations, any row count), the standalone
// block-Hadamard rotation, the output-head argmax and the streaming-read reference.
#include "vg_device.h"
#include "vg_launch.h"

namespace vg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int VALU_THREADS = 256;
constexpr int VALU_WK = 2048;   // K per LDS window
// In LDS every word's K values (32 or 16) are followed by 4 unused floats, so the parts of a
// row, which read their words' values at the same offset at the same time, fall on different
// bank quads instead of all on one (a word is 128 or 64 bytes wide).
constexpr int VALU_PAD = 4;
constexpr int VALU_PITCH = VALU_WK + VALU_WK / 16 * VALU_PAD;   // floats per staged row
template <int WK>
__device__ __forceinline__ int xs_col(int k) { return k + (k / WK) * VALU_PAD; }
constexpr int MAXM = 8;
constexpr int VG_MAX_ROWS_DEV = 8;   // counter m (row m, m < 8) and counter 8 (finished rows)
// Each counter has its own 128-byte line: all of a row's chunks update it, and counters
// sharing a line would serialize every row's updates behind each other.
constexpr int ARG_CTR_STRIDE = 32;   // u32 elements

__device__ __forceinline__ float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ float x_at(const void* x, int xt, size_t idx) {
  if (xt == 0) return static_cast<const float*>(x)[idx];
  const uint32_t h = static_cast<const uint16_t*>(x)[idx];
  return xt == 2 ? __uint_as_float(h << 16) : h2f(h);
}

struct ValuArgs {
  const void* x;
  int xt;
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
  float* y;
  int M, K, N;
  int had_block;            // rotated format: 64, 128 or 256
  const uint32_t* signs;    // rotated format: optional sign bits [K/32]
  bool sbi;                 // scales holds interleaved (scale, bias) words, biases unused
};

__device__ __forceinline__ float had_norm(int block) {
  return block == 64 ? 0.125f : (block == 256 ? 0.0625f : 0.08838834764831845f);   // 1/sqrt(block)
}

// In-place unnormalized Walsh-Hadamard transform of the `block`-blocks of the first `len`
// elements of each staged row (len a multiple of block), butterfly stage by stage.
template <int WK>
__device__ void lds_fwht(float* xs, int rows, int len, int block) {
  const int pairs = rows * len / 2, half = block / 2;
  for (int h = 1; h < block; h <<= 1) {
    for (int p = threadIdx.x; p < pairs; p += blockDim.x) {
      const int m = p / (len / 2), q = p - m * (len / 2);
      const int blk = q / half, r = q - blk * half;          // block/2 butterflies per block
      const int lo = (r / h) * (2 * h) + (r % h);
      float* b = xs + m * VALU_PITCH;
      const int i0 = xs_col<WK>(blk * block + lo), i1 = xs_col<WK>(blk * block + lo + h);
      const float a0 = b[i0], a1 = b[i1];
      b[i0] = a0 + a1;
      b[i1] = a0 - a1;
    }
    __syncthreads();
  }
}

// VALU kernel: exact fp32 dequantization and fp32 fused multiply-adds.  A workgroup takes
// VALU_ROWS output rows; the VALU_PARTS threads of a row split its words round-robin (part
// p takes words p, p + VALU_PARTS, ...), so neighbouring threads read neighbouring words of
// a row and threads of equal part read the same activations (an LDS broadcast).  The parts
// are added in part order through LDS, so results do not depend on timing.
//
// The kernel is latency-bound at the sizes it serves (few workgroups, one wave per SIMD), so
// every thread issues all of its loads of a window at once: its weight words, scales and
// biases, then its share of the activation window.  A workgroup computes MM rows, rows
// m0 = MM * blockIdx.y onward: all M rows (MM = M rounded up to 1, 2, 4 or 8) or, when the
// grid leaves CUs idle, two rows each with the row pairs spread over blockIdx.y.  Staged
// rows past M are zeros, so the row loops carry no run-time bounds.
constexpr int VALU_PARTS = 16;
constexpr int VALU_ROWS = VALU_THREADS / VALU_PARTS;

template <int XT>
__device__ __forceinline__ float load_x(const void* x, size_t idx) {
  if constexpr (XT == 0) return static_cast<const float*>(x)[idx];
  const uint32_t h = static_cast<const uint16_t*>(x)[idx];
  if constexpr (XT == 2) return __uint_as_float(h << 16);
  return h2f(h);
}

// A thread's share of an activation window: elements k = tid + i * VALU_THREADS of rows
// m0 .. m0 + MM - 1, all loads issued back to back (rows past M and k >= len read as zeros,
// without a load).
constexpr int VALU_NI = VALU_WK / VALU_THREADS;
template <int XT, int MM>
__device__ __forceinline__ void load_window(const void* x, int M, int m0, int K, int k0, int len,
                                            float (&v)[MM][VALU_NI]) {
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int i = 0; i < VALU_NI; ++i) {
      const int k = threadIdx.x + i * VALU_THREADS;
      v[m][i] = (m0 + m < M && k < len) ? load_x<XT>(x, (size_t)(m0 + m) * K + k0 + k) : 0.0f;
    }
}

template <int WK, int MM>
__device__ __forceinline__ void store_window(const float (&v)[MM][VALU_NI], int len, float* xs) {
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int i = 0; i < VALU_NI; ++i) {
      const int k = threadIdx.x + i * VALU_THREADS;
      if (k < len) xs[m * VALU_PITCH + xs_col<WK>(k)] = v[m][i];
    }
}

template <int FMT, int XT, int MM>
__global__ __launch_bounds__(VALU_THREADS) void vg_valu(ValuArgs A) {
  __shared__ float xs[MAXM * VALU_PITCH];
  __shared__ float red[VALU_ROWS][VALU_PARTS][MM + 1];   // +1: rows of parts on different banks
  constexpr int G = fmt_one_bit(FMT) ? 128 : 64;
  constexpr int WK = fmt_one_bit(FMT) ? 32 : 16;        // K per word
  constexpr int NWJ = VALU_WK / WK / VALU_PARTS;         // words per thread per full window
  constexpr bool BIAS = FMT != SIGN1;
  const int part = threadIdx.x % VALU_PARTS, lr = threadIdx.x / VALU_PARTS;
  const int m0 = (int)blockIdx.y * MM;                   // this workgroup's first row
  const int n = blockIdx.x * VALU_ROWS + lr;
  const int nl = min(n, A.N - 1);                        // rows past N compute row N-1, unstored
  const size_t wrow = (size_t)nl * (A.K / WK), grow = (size_t)nl * (A.K / G);
  float acc[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
  for (int k0 = 0; k0 < A.K; k0 += VALU_WK) {
    const int len = min(VALU_WK, A.K - k0), nw = len / WK;
    uint32_t word[NWJ], scb[NWJ], bib[NWJ];             // raw: converted where used
#pragma unroll
    for (int j = 0; j < NWJ; ++j) {                      // clamped: every load in bounds
      const int wi = min(part + j * VALU_PARTS, nw - 1);
      const int k = k0 + WK * wi;
      word[j] = A.w[wrow + k / WK];
      if (BIAS && A.sbi) {
        const uint32_t sb = reinterpret_cast<const uint32_t*>(A.scales)[grow + k / G];
        scb[j] = sb & 0xFFFFu;
        bib[j] = sb >> 16;
      } else {
        scb[j] = A.scales[grow + k / G];
        bib[j] = BIAS ? A.biases[grow + k / G] : 0u;
      }
    }
    float xv[MM][VALU_NI];
    load_window<XT, MM>(A.x, A.M, m0, A.K, k0, len, xv);
    __syncthreads();                                     // the previous window is consumed
    store_window<WK, MM>(xv, len, xs);
    __syncthreads();
    if constexpr (FMT == HAD2) {
      if (A.signs) {
        for (int e = threadIdx.x; e < MM * len; e += VALU_THREADS) {
          const int m = e / len, kk = e - m * len, k = k0 + kk;
          float* p = xs + m * VALU_PITCH + xs_col<WK>(kk);
          if ((A.signs[k >> 5] >> (k & 31)) & 1u) *p = -*p;
        }
        __syncthreads();
      }
      lds_fwht<WK>(xs, MM, len, A.had_block);
      const float nrm = had_norm(A.had_block);
      for (int e = threadIdx.x; e < MM * len; e += VALU_THREADS) {
        const int m = e / len, kk = e - m * len;
        xs[m * VALU_PITCH + xs_col<WK>(kk)] *= nrm;
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NWJ; ++j) {
      const int wi = part + j * VALU_PARTS;
      if (wi < nw) {
        const float* xw = xs + (WK + VALU_PAD) * wi;
        const float scj = h2f(scb[j]), bij = BIAS ? h2f(bib[j]) : 0.0f;
        if constexpr (fmt_one_bit(FMT)) {
          const float won = FMT == AFFINE1 ? scj + bij : scj;    // one fp32 rounding at most
          const float woff = FMT == AFFINE1 ? bij : -scj;
#pragma unroll 4
          for (int bit = 0; bit < 32; ++bit) {
            const float wv = ((word[j] >> bit) & 1u) ? won : woff;
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[m] = __builtin_fmaf(xw[m * VALU_PITCH + bit], wv, acc[m]);
          }
        } else {
#pragma unroll 4
          for (int c = 0; c < 16; ++c) {
            const float wv = (float)((word[j] >> (2 * c)) & 3u) * scj + bij;   // one fp32 rounding at most
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[m] = __builtin_fmaf(xw[m * VALU_PITCH + c], wv, acc[m]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MM; ++m) red[lr][part][m] = acc[m];
  __syncthreads();
  // Thread (lr, m) adds row m0 + m's parts in part order.
  if (part < MM && m0 + part < A.M && n < A.N) {
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < VALU_PARTS; ++q) sum += red[lr][q][part];
    A.y[(size_t)(m0 + part) * A.N + n] = sum;
  }
}

// rows_per_wg: 2 when the row pairs go to separate workgroups, else 0 (all rows in one)
template <int FMT, int XT>
static void launch_valu_m(const ValuArgs& A, dim3 grid, int rows_per_wg, hipStream_t s) {
  if (A.M <= 1) hipLaunchKernelGGL((vg_valu<FMT, XT, 1>), grid, dim3(VALU_THREADS), 0, s, A);
  else if (A.M <= 2 || rows_per_wg == 2) hipLaunchKernelGGL((vg_valu<FMT, XT, 2>), grid, dim3(VALU_THREADS), 0, s, A);
  else if (A.M <= 4) hipLaunchKernelGGL((vg_valu<FMT, XT, 4>), grid, dim3(VALU_THREADS), 0, s, A);
  else hipLaunchKernelGGL((vg_valu<FMT, XT, 8>), grid, dim3(VALU_THREADS), 0, s, A);
}

template <int FMT>
static hipError_t launch_valu_x(const ValuArgs& A, dim3 grid, int rows_per_wg, hipStream_t s) {
  switch (A.xt) {
    case 0: launch_valu_m<FMT, 0>(A, grid, rows_per_wg, s); break;
    case 1: launch_valu_m<FMT, 1>(A, grid, rows_per_wg, s); break;
    case 2: launch_valu_m<FMT, 2>(A, grid, rows_per_wg, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// A grid too small to fill the CUs with all rows per workgroup (the kernel is latency-bound
// there, and a workgroup's time grows with its rows) gives each row pair its own
// workgroups: the packed words are then read once per pair, a small cost at these sizes.
hipError_t launch_valu(const GemmCall& c, const DeviceInfo& dev) {
  if (c.M < 1 || c.M > MAXM || c.N < 1) return hipErrorInvalidValue;
  ValuArgs A{c.x, c.xt, c.w, c.scales, c.biases, c.y, c.M, c.K, c.N, c.had_block, c.signs, c.sbi};
  dim3 grid((c.N + VALU_ROWS - 1) / VALU_ROWS);
  int rows_per_wg = 0;
  const int pairs = (c.M + 1) / 2;
  if (c.M > 2 && (long long)grid.x * pairs <= dev.cu_count) {
    grid.y = pairs;
    rows_per_wg = 2;
  }
  switch (c.fmt) {
    case SIGN1: return launch_valu_x<SIGN1>(A, grid, rows_per_wg, c.stream);
    case AFFINE2: return launch_valu_x<AFFINE2>(A, grid, rows_per_wg, c.stream);
    case HAD2: return launch_valu_x<HAD2>(A, grid, rows_per_wg, c.stream);
    case AFFINE1: return launch_valu_x<AFFINE1>(A, grid, rows_per_wg, c.stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------------------
// Interleaved (scale, bias) layout of the affine formats' group metadata: one word per
// group, the scale in the low half.  Built once when the weights are loaded; the GEMMs then
// fetch a lane's scales and biases with one load instead of one per array.
__global__ __launch_bounds__(256) void vg_pack_scale_bias_kernel(const uint16_t* s, const uint16_t* b,
                                                                long long count, uint32_t* out) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count; i += stride)
    out[i] = (uint32_t)s[i] | ((uint32_t)b[i] << 16);
}

hipError_t launch_pack_scale_bias(const uint16_t* s, const uint16_t* b, long long count, uint32_t* out,
                                  hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const long long blocks = (count + 255) / 256;
  hipLaunchKernelGGL(vg_pack_scale_bias_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st,
                     s, b, count, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Standalone rotation: x_out = x * blockdiag(H_128 / sqrt(128)), one quad of lanes per
// (row, block), each lane 32 consecutive elements; same butterfly scheme as the fused
// GEMM prologue.
template <int CTRL>
__device__ __forceinline__ float dpp_quad_aux(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__global__ __launch_bounds__(256) void vg_hadamard_kernel(const void* x, int xt, int M, int K, int block,
                                                         const uint32_t* signs, float* out) {
  const int lanes = block / 32, stages = lanes == 2 ? 1 : (lanes == 4 ? 2 : 3);
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int nblocks = M * (K / block);
  const int bid = gt / lanes, bl = gt % lanes;
  if (bid >= nblocks) return;          // whole blocks leave together (lanes | 256)
  const int m = bid / (K / block), blk = bid - m * (K / block);
  const int k0 = blk * block + bl * 32;
  const size_t base = (size_t)m * K + k0;
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = x_at(x, xt, base + e);
  if (signs) {
    const uint32_t sw = signs[k0 >> 5];
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((sw >> e) & 1u) << 31));
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if ((e & h) == 0) { const float a = v[e], b = v[e + h]; v[e] = a + b; v[e + h] = a - b; }
  // cross-lane stages, upper results negated (the final sign is the parity of bl)
  const float c1 = (bl & 1) ? -1.0f : 1.0f, c2 = (bl & 2) ? -1.0f : 1.0f, c3 = (bl & 4) ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = __builtin_fmaf(c1, dpp_quad_aux<0xB1>(v[e]), v[e]);
  if (stages >= 2) {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = __builtin_fmaf(c2, dpp_quad_aux<0x4E>(v[e]), v[e]);
  }
  if (stages >= 3) {
#pragma unroll
    for (int e = 0; e < 32; ++e)
      v[e] = __builtin_fmaf(c3, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v[e]), 0x101F)), v[e]);
  }
  const float sg = (__builtin_popcount(bl) & 1) ? -1.0f : 1.0f;
  const float sc = sg * had_norm(block);
#pragma unroll
  for (int e = 0; e < 32; ++e) out[base + e] = v[e] * sc;
}

hipError_t launch_hadamard(const void* x, int xt, int M, int K, int block, const uint32_t* signs, float* out,
                           hipStream_t s) {
  const int threads = (block / 32) * M * (K / block);
  hipLaunchKernelGGL(vg_hadamard_kernel, dim3((threads + 255) / 256), dim3(256), 0, s, x, xt, M, K, block, signs, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Per-row argmax of fp32 logits over the whole chip, then (optionally) greedy acceptance of
// a drafted block.  Block (c, m) scans columns [c*ARG_CHUNK, ...) of row m and parks its
// best (value, column) as one 64-bit key that orders like (value, -column): the value's bits
// made order-preserving in the high half (-0 taken as +0), the complemented column in the
// low half, NaN never entering.  The last chunk of a row to arrive takes the maximum over
// the row's keys, and the last row to finish counts the leading rows whose argmax equals
// the drafted token ("dflash-mlx-bonsai2" README, "Verify it yourself": greedy acceptance
// and argmax parity).  Lowest column on ties; a row of only NaN gives 0.  The parked keys
// and the counters are agent-scope atomic accesses (they bypass the per-XCD L2 caches), so
// no device-wide fence is needed; each key has its own 128-byte line.
constexpr int ARG_THREADS = 256;
constexpr int ARG_PER_THREAD = 8;                          // loads in flight per thread
constexpr int ARG_CHUNK = ARG_THREADS * ARG_PER_THREAD;    // columns per block
constexpr int ARG_KEY_STRIDE = 16;                         // u64 elements between parked keys

__device__ __forceinline__ unsigned long long arg_key_aux(float v, int n) {
  const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // orders like v
  return ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)n;
}

// Block-wide maximum of the threads' keys: across each wave by shuffles, then the four
// waves' maxima through LDS.
__device__ __forceinline__ unsigned long long arg_block_max(unsigned long long* sk, unsigned long long k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  if ((threadIdx.x & 63) == 0) sk[threadIdx.x >> 6] = k;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < ARG_THREADS / 64; ++w) k = sk[w] > k ? sk[w] : k;
  return k;
}

__global__ __launch_bounds__(ARG_THREADS) void vg_argmax_kernel(const float* y, int M, int N, int32_t* idx,
                                                              const int32_t* draft, int32_t* accepted,
                                                              unsigned long long* pkey, uint32_t* counters) {
  __shared__ unsigned long long sk[ARG_THREADS / 64];
  __shared__ uint32_t last;
  const int c = blockIdx.x, m = blockIdx.y, C = gridDim.x;
  const float* row = y + (size_t)m * N;
  const int n0 = c * ARG_CHUNK + threadIdx.x;
  float v[ARG_PER_THREAD];
#pragma unroll
  for (int e = 0; e < ARG_PER_THREAD; ++e) {
    const int n = n0 + e * ARG_THREADS;
    v[e] = n < N ? row[n] : __builtin_nanf("");
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int e = 0; e < ARG_PER_THREAD; ++e) {
    if (v[e] == v[e]) {
      const unsigned long long k = arg_key_aux(v[e], n0 + e * ARG_THREADS);
      best = k > best ? k : best;
    }
  }
  best = arg_block_max(sk, best);
  if (threadIdx.x == 0) {
    __hip_atomic_store(pkey + (size_t)(m * C + c) * ARG_KEY_STRIDE, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the key has landed
    last = __hip_atomic_fetch_add(counters + m * ARG_CTR_STRIDE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(C - 1);
  }
  __syncthreads();
  if (!last) return;
  // last chunk of row m to finish: the maximum over the row's C keys
  best = 0ull;
  for (int k = threadIdx.x; k < C; k += ARG_THREADS) {
    const unsigned long long pk =
        __hip_atomic_load(pkey + (size_t)(m * C + k) * ARG_KEY_STRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    best = pk > best ? pk : best;
  }
  __syncthreads();   // sk is reused
  best = arg_block_max(sk, best);
  if (threadIdx.x != 0) return;
  const int32_t am = best == 0ull ? 0 : (int32_t)~(uint32_t)best;
  __hip_atomic_store(idx + m, am, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(counters + m * ARG_CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (draft == nullptr) return;
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (__hip_atomic_fetch_add(counters + VG_MAX_ROWS_DEV * ARG_CTR_STRIDE, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)(M - 1))
    return;
  // last row to finish: the drafted prefix the target agrees with
  int L = 0;
  while (L < M && __hip_atomic_load(idx + L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == draft[L]) ++L;
  accepted[0] = L;
  __hip_atomic_store(counters + VG_MAX_ROWS_DEV * ARG_CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int argmax_chunks(int N) { return (N + ARG_CHUNK - 1) / ARG_CHUNK; }

// The fused argmax's last step, after the GEMM on the same stream (whose end makes its keys
// visible): wave m folds row m's keys of all G workgroups (a key orders like (value,
// -column)), with its lanes' loads in flight together, and writes idx[m].  With a draft, the
// waves' verdicts meet in LDS and wave 0 counts the leading rows that agree.
__global__ __launch_bounds__(64 * FUSED_KEYS) void vg_argmax_keys_kernel(const unsigned long long* keys, int G,
                                                                          int M, int32_t* idx, const int32_t* draft,
                                                                          int32_t* accepted) {
  __shared__ int agree[FUSED_KEYS];
  const int m = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (m < M) {
    const int want = draft != nullptr && lane == 0 ? draft[m] : 0;   // read before the keys land
    unsigned long long k = 0ull;
    for (int g0 = 0; g0 < G; g0 += 4 * 64) {
      unsigned long long v[4];
      // lanes past the last workgroup read its key again (the maximum does not change), so
      // the loads need no branch and all four are in flight together
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = keys[(size_t)min(g0 + 64 * j + lane, G - 1) * FUSED_KEYS + m];
#pragma unroll
      for (int j = 0; j < 4; ++j) k = v[j] > k ? v[j] : k;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(k, off);
      k = o > k ? o : k;
    }
    const int id = k == 0ull ? 0 : (int)~(uint32_t)k;
    if (lane == 0) {
      idx[m] = id;
      agree[m] = id == want;
    }
  }
  if (draft == nullptr) return;   // uniform over the workgroup
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // the accepted prefix: the rows before the first that disagrees
  const unsigned long long bad = __ballot(lane < M && !agree[lane < M ? lane : 0]);
  if (lane == 0) accepted[0] = bad == 0ull ? M : __builtin_ctzll(bad);
}

hipError_t launch_argmax_keys(const unsigned long long* keys, int G, int M, int32_t* idx, const int32_t* draft,
                              int32_t* accepted, hipStream_t s) {
  if (M < 1 || M > FUSED_KEYS || G < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vg_argmax_keys_kernel, dim3(1), dim3(64 * FUSED_KEYS), 0, s, keys, G, M, idx, draft, accepted);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* y, int M, int N, int32_t* idx, const int32_t* draft, int32_t* accepted,
                         unsigned long long* pkey, uint32_t* counters, hipStream_t s) {
  hipLaunchKernelGGL(vg_argmax_kernel, dim3(argmax_chunks(N), M), dim3(ARG_THREADS), 0, s, y, M, N, idx, draft,
                     accepted, pkey, counters);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Streaming read of a buffer, for the measurement's achievable-bandwidth reference: every
// byte is read once with 16-byte non-temporal loads, U in flight per thread, and folded
// into one word per workgroup so the loads cannot be elided.  The loads in flight per
// thread and the workgroups per CU are parameters, so the reference can be swept.
constexpr int STREAM_THREADS = 256;
constexpr int STREAM_MAX_WGS_PER_CU = 32;
template <int U>
__global__ __launch_bounds__(STREAM_THREADS) void vg_stream_read_kernel(const u32x4* buf, size_t n16, uint32_t* sink) {
  __shared__ uint32_t part[STREAM_THREADS / 64];
  const size_t stride = (size_t)gridDim.x * STREAM_THREADS;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * STREAM_THREADS + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

int stream_read_blocks(const DeviceInfo& dev) { return dev.cu_count * STREAM_MAX_WGS_PER_CU; }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int loads_in_flight, int wgs_per_cu,
                              const DeviceInfo& dev, hipStream_t s) {
  if (wgs_per_cu < 1 || wgs_per_cu > STREAM_MAX_WGS_PER_CU) return hipErrorInvalidValue;
  const dim3 grid(dev.cu_count * wgs_per_cu), block(STREAM_THREADS);
  const u32x4* b = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  switch (loads_in_flight) {
    case 1: hipLaunchKernelGGL(vg_stream_read_kernel<1>, grid, block, 0, s, b, n16, sink); break;
    case 2: hipLaunchKernelGGL(vg_stream_read_kernel<2>, grid, block, 0, s, b, n16, sink); break;
    case 4: hipLaunchKernelGGL(vg_stream_read_kernel<4>, grid, block, 0, s, b, n16, sink); break;
    case 8: hipLaunchKernelGGL(vg_stream_read_kernel<8>, grid, block, 0, s, b, n16, sink); break;
    case 16: hipLaunchKernelGGL(vg_stream_read_kernel<16>, grid, block, 0, s, b, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vg
