// vg_kernels.hip -- few-row quantized verify GEMM kernels for MI355X (gfx950).
//
// y[M, N] = x[M, K] * W^T for M <= 8 drafted rows and packed 1-bit sign (g128) or 2-bit
// affine (g64) weights, optionally after a block-128 Hadamard rotation of x.  Each packed
// weight is read from HBM once and decoded once, straight into MFMA operand registers,
// and multiplied against every drafted row ("Ishizuki" README, "Kernels written for the
// verify"; "dflash-mlx-bonsai2" README, "What this fork adds").
//
// Work decomposition (MFMA variants)
//   * One workgroup (8 waves) per CU owns a contiguous, balanced range of output rows;
//     rows are grouped in tiles of 16 (the MFMA N dimension).  A "unit" is one tile times
//     one K-step of 1024 (8 sign groups or 16 affine groups).  Per unit each lane loads
//     GL consecutive groups of one row in single wide loads (codes, then the scales and
//     biases of those groups: one load per array, or one load of the interleaved
//     scale-and-bias pairs), so a row's unit is fetched by 4 lanes as 256 contiguous
//     bytes of codes.  Every wave keeps PREF units in flight in a register ring (two for
//     the 1-bit formats, whose units are half as large, one for the 2-bit formats).
//   * K is processed in windows.  Per window the workgroup first loads its activations,
//     then stages them into LDS, already in the operand layout the unpacked codes need
//     (and rotated, for the Hadamard format), together with per-(group, row) correction
//     sums.  Weight loads never go out ahead of a wave's activation loads: loads leave a
//     CU in order, and a burst of weight loads ahead of the activations would delay every
//     MFMA behind it.  The 8-row variant issues each wave's first units as soon as that
//     wave's activations have landed, the others once the staging is done.  The window's
//     units are split evenly across the 8 waves in tile-major order; partial tiles are
//     reduced through LDS in a fixed order, so results are deterministic.
//   * MFMA rows: the 16 A rows are split into independent row-blocks, each fed only by
//     one lane-group's K slots.  Mode Q: 4 blocks of 4 rows (M <= 4), each lane-group
//     decodes its own quantization group.  Mode H: 2 blocks of 8 rows (M <= 8), lane-group
//     pairs share a group after one permlane16 swap of two words.  Every accumulator
//     register therefore holds one quantization group's dot products, and the per-group
//     scale (and bias) is applied once per group in fp32.  The lanes whose A row carries
//     no drafted row feed zeros: a zero row in LDS, or for 1-bit codes at 8 rows operand
//     registers cleared once per launch, their reads masked off.
//   * K split across workgroups (tall K, or the rotated format): each slice
//     parks its partial outputs and the last slice of a row group to arrive adds them in
//     slice order.
//   * The output-head epilogue (verify_gemm_argmax, one K slice): every row's argmax over
//     the workgroups' columns as one 64-bit maximum per row (fused_argmax).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "vg_device.h"
#include "vg_launch.h"

namespace vg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum XType : int { XF32 = 0, XF16 = 1, XBF16 = 2 };

constexpr int NW = 8;               // waves per workgroup
static_assert(NW <= 16, "split-tile records hold a 16-bit wave mask");
constexpr int NTHREADS = NW * 64;
constexpr int MAXM = 8;

template <int FMT> struct Fmt;
// GL: consecutive quantization groups each lane loads per unit (16*GL bytes of codes and
// 2*GL bytes of scales in single loads, 64*GL contiguous bytes per row and unit); a unit
// covers 4*GL groups = 1024 K for both formats.
template <> struct Fmt<SIGN1> {
  static constexpr int G = 128, WORD_K = 32, PAIRS = 16, NQ = 4, GL = 2;
  static constexpr int WB = 64;           // LDS bytes of one word's operand window
  static constexpr int GS = 4 * WB + 16;  // LDS bytes per group (+16 pad vs bank conflicts)
  static constexpr bool AFFINE = false;   // a bias per group
  static constexpr bool ONE_BIT = true;   // sign-bit decode (else 2-bit codes)
};
template <> struct Fmt<AFFINE1> : Fmt<SIGN1> {
  static constexpr bool AFFINE = true;
};
template <> struct Fmt<AFFINE2> {
  static constexpr int G = 64, WORD_K = 16, PAIRS = 8, NQ = 2, GL = 4;
  static constexpr int WB = 32;
  static constexpr int GS = 4 * WB + 16;
  static constexpr bool AFFINE = true;
  static constexpr bool ONE_BIT = false;
};
template <> struct Fmt<HAD2> : Fmt<AFFINE2> {};

__host__ __device__ constexpr int fmt_group(int fmt) { return fmt_one_bit(fmt) ? 128 : 64; }
__host__ __device__ constexpr int fmt_gs(int fmt) { return fmt_one_bit(fmt) ? 4 * 64 + 16 : 4 * 32 + 16; }
__host__ __device__ constexpr int fmt_word_k(int fmt) { return fmt_one_bit(fmt) ? 32 : 16; }
__host__ __device__ constexpr int fmt_gps(int fmt) { return fmt_one_bit(fmt) ? 8 : 16; }   // groups per K-step
__host__ __device__ constexpr int fmt_gl(int fmt) { return fmt_one_bit(fmt) ? 2 : 4; }     // Fmt<>::GL
constexpr int KSTEP = 1024;   // K per unit, both formats
// bf16 activations meet 1-bit codes in bf16 MFMAs (the codes decode to bf16 exactly);
// against 2-bit codes, and for the rotated format, each activation row is rescaled by a
// power of two into fp16 first.
__host__ __device__ constexpr bool bf16_codes(int fmt, int xt) { return fmt_one_bit(fmt) && xt == XBF16; }
__host__ __device__ constexpr bool x_rescaled(int fmt, int xt) { return fmt == HAD2 || (xt == XBF16 && !fmt_one_bit(fmt)); }

// LDS carve-up (byte offsets), computed identically on host and device.
//   a:  activation operand rows 0..M-1 of the window, then row M, all zeros (read by the
//       lanes whose operand row carries no drafted row)
//   e:  fp32 per-(group, row) offset sums, the accumulators' initial values
//   xp: 2-bit formats: per (row, lane-group quad of GL groups) the group sums / 64 as
//       fp16 hi parts then lo parts (16 bytes), rows 0..M-1 and a zero row M
//   job (first 128 bytes): grouped expert verify, the workgroup's job (find_job)
constexpr int JOB_BYTES = 128;
struct LdsLayout {
  int a_off, e_off, xp_off, xp_pitch, ytile_off, slot_off, row_off, flag_off, red_off, total;
  LdsLayout() = default;
  __host__ __device__ LdsLayout(int fmt, int M, int win_steps, int tiles_max) {
    const int groups = win_steps * fmt_gps(fmt);
    const int pitch = groups * fmt_gs(fmt) + 16;   // must equal MfmaArgs::a_pitch
    a_off = JOB_BYTES;
    e_off = a_off + (M + 1) * pitch;
    xp_off = e_off + groups * MAXM * 4;
    xp_pitch = (groups / fmt_gl(fmt)) * 16 + 16;
    ytile_off = xp_off + (fmt == SIGN1 ? 0 : (M + 1) * xp_pitch);   // every other format has biases
    slot_off = ytile_off + tiles_max * MAXM * 16 * 4;
    row_off = slot_off + NW * 2 * MAXM * 16 * 4;
    flag_off = row_off + 2 * MAXM * 4;
    red_off = flag_off + 16;   // split tiles of the window, two words per wave boundary
    total = red_off + NW * 8;
  }
};

struct MfmaArgs {
  const void* x;
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
  float* y;
  int M, K, N;
  int win_steps;   // K-steps (of KSTEP) per staging window
  int tiles_max;   // ytile capacity
  int a_pitch;     // LDS bytes per activation row in a window
  uint32_t mask[8];   // code-extraction masks per bit position (see vg_device.h)
  uint32_t magic[8];  // magic pairs per bit position (fp16; bf16 for 1-bit codes with bf16 x)
  int rg, ks;         // row groups x K slices; workgroup b takes row group b / ks, slice b % ks
  // Per-call constants the host works out once, so the workgroups' shared scalar unit does
  // not (eight waves each running the same integer divisions cost about a microsecond):
  int rq, rrem;        // N = rq * rg + rrem
  uint32_t ks_magic;   // ks >= 2: ceil(2^32 / ks), n / ks = mulhi(n, ks_magic) for n * ks < 2^32
  uint32_t ws_magic;   // win_steps >= 2: the same for win_steps
  LdsLayout lay;       // the LDS carve-up at M (a grouped verify's jobs work out their own)
  int had_stages;     // rotated format: log2(block / 32) cross-lane butterfly stages
  float had_scale;    // 1 / sqrt(block)
  const uint32_t* signs;  // rotated format: optional sign bits [K/32] (bit set: negate x[:, k])
  float* part;        // ks > 1: partial outputs [ks][M][N]
  uint32_t* counters; // ks > 1: arrivals per row group (zero between calls), row group r's at
                      // counters[r * SPLIT_CTR_STRIDE]
  // Grouped expert verify (route non-null, ks = 1): route [M, topk] names the expert of
  // each (row, slot); values outside 0..E-1 mark unused slots.  Each workgroup groups the
  // routing by expert into jobs of at most cap rows and takes one row group of one job
  // (find_job); rg is then the fewest row groups per job the plan sized the LDS for.
  // Expert e's codes start e * w_estride bytes into w, its scales and biases e * s_estride
  // bytes into scales and biases; y is [M * topk, N].
  const int32_t* route;
  int topk, E, cap;
  long long w_estride, s_estride;
  // Fused argmax (plain calls with ks = 1; idx null otherwise): the workgroup's largest key
  // of each row goes to amax_key[FUSED_KEYS * blockIdx.x + m] (fused_argmax), and the
  // launch after the GEMM turns them into idx [M] and, with draft non-null, accepted[0] (the
  // number of leading rows whose argmax equals draft[m]).  `reserved` is unused: it keeps the
  // argument block at the size and layout the kernels were timed with.
  int32_t* idx;
  const int32_t* draft;
  int32_t* accepted;
  unsigned long long* amax_key;
  uint32_t* reserved;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}
// CTRL 0xB1: quad_perm [1,0,3,2] (partner lane ^1); 0x4E: quad_perm [2,3,0,1] (lane ^2).
// Every lane of a quad permutation has a source, so no old value is kept (bound_ctrl):
// the compiler can then fold the move into the arithmetic that consumes it as a DPP operand.
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Lane l ^ 4 within groups of 32 lanes (ds_swizzle, bit-mask mode: and 0x1f, xor 4).
__device__ __forceinline__ float swizzle_xor4(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101F));
}

// Fast Walsh-Hadamard transform of a block of 32 * 2^stages elements (64, 128 or 256) held
// by 2^stages consecutive lanes, 32 fp32 values per lane, lane b of the block holding
// block elements 32b .. 32b+31.  Five butterfly stages run inside each lane's registers,
// `stages` across lanes (partners b ^ 1, b ^ 2 by DPP, b ^ 4 by swizzle).  Each cross-lane
// stage is one fused multiply-add that leaves the upper results negated; the final sign of
// each lane, (-1)^popcount(b), is returned so the caller can fold it into its scale.
// Unnormalized: out[k] = sign * sum_j (-1)^popcount(k & j) in[j].
__device__ __forceinline__ float fwht_lanes(float v[32], int block_lane, int stages) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if ((e & h) == 0) {
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  if (stages >= 1) {
    const float c1 = (block_lane & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = __builtin_fmaf(c1, dpp_quad<0xB1>(v[e]), v[e]);
  }
  if (stages >= 2) {
    const float c2 = (block_lane & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = __builtin_fmaf(c2, dpp_quad<0x4E>(v[e]), v[e]);
  }
  if (stages >= 3) {
    const float c3 = (block_lane & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = __builtin_fmaf(c3, swizzle_xor4(v[e]), v[e]);
  }
  return (__builtin_popcount(block_lane & ((1 << stages) - 1)) & 1) ? -1.0f : 1.0f;
}

// Workgroup barrier for hand-offs through LDS.  The fences order LDS accesses only, so a
// wave waits for its own LDS operations but not for its global loads: a __syncthreads
// would also drain every weight load in flight and serialize the prefetch with it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Loads 32 consecutive activations of row m starting at k0 as fp32 (XT: F16 or BF16).
template <int XT>
__device__ __forceinline__ void load_x32_f32(const void* x, int K, int m, int k0, float v[32]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + (size_t)m * K + k0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 d = p[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = d[i] & 0xFFFFu, hi = d[i] >> 16;
      v[8 * q + 2 * i] = XT == XBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
      v[8 * q + 2 * i + 1] = XT == XBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Activation staging for one window: x[m, k0 .. k0 + WK) -> LDS operand layout + sums.
//
// Operand layout: for each row m, group gr and word w of the group, the word's window of
// WORD_K activations is stored as PAIRS dwords, dword j = (x[k_j], x[k_j + WORD_K/2]) in
// fp16, k_j = j-th K index of the window, i.e. exactly the pairing of unpacked code
// registers (bits p and p+16).  An MFMA operand of 4 consecutive registers therefore maps
// to 16 contiguous bytes.
// Sums per (group, row), fp32, computed from the same operand values:
//   1-bit:  E = sum_k a_k * (BETA_k + 1)          (stored negated)
//   2-bit:  R = sum_k a_k * BETA_k (stored negated),  X = sum_k a_k
// The activations a are x * f (f a per-row power of two chosen so the fp16 values cannot
// overflow; f = 1 for fp16 input without rotation and for bf16 input against 1-bit codes,
// which stays bf16), rotated first for the Hadamard format.
// The staging is split in two so the activation loads can be issued before a wave's
// weight prefetch: loads enter the memory pipeline in order, and staged behind the weight
// burst they would delay every workgroup's first MFMA by that whole burst.
constexpr int MAXT = 3;   // activation chunks (32 K of one row) per thread and window
// Thread tid's chunk in staging round j (MAXT * NTHREADS when it has none).  The chunks go
// to all NTHREADS threads in turn, or with SIX to the first six waves only (the launch
// takes SIX for at most NTHREADS chunks, which MAXT rounds of six waves cover).
template <bool SIX>
__device__ __forceinline__ int stage_task(int tid, int j) {
  if constexpr (SIX) return tid < 6 * 64 ? tid + j * (6 * 64) : MAXT * NTHREADS;
  else return tid + j * NTHREADS;
}
struct XStage {
  u32x4 d[MAXT][4];       // raw fp16/bf16 bits of 32 consecutive activations
  int m[MAXT], c[MAXT];   // the chunk's row and its index within the row's window
};

template <int XT, bool SIX>
// xmap: the x row of each row (grouped expert verify), or null for x rows 0..M-1.
__device__ __forceinline__ void stage_load(const MfmaArgs& A, int M, const int* xmap, int k0, int WK, XStage& xs) {
  const int nchunks = WK / 32, ntask = M * nchunks;
  // row = t / nchunks = (t / 32) / (WK / 1024) for t < MAXT * NTHREADS, by a float
  // reciprocal: (n + 1/2) / s lies at least 1/(2s) from an integer, far beyond the
  // rounding of the product for n < 128 and s <= 64
  const float inv_steps = 1.0f / (float)(WK / KSTEP);
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    const int t = stage_task<SIX>((int)threadIdx.x, j);
    const int m = (int)(((float)(t >> 5) + 0.5f) * inv_steps), c = t - m * nchunks;
    xs.m[j] = m;
    xs.c[j] = c;
    if (t < ntask) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(A.x) + (size_t)(xmap ? xmap[m] : m) * A.K + k0 + 32 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) xs.d[j][q] = p[q];
    }
  }
}

__device__ __forceinline__ void chunk_halves(const XStage& xs, int j, uint32_t hv[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[8 * q + 2 * i] = xs.d[j][q][i] & 0xFFFFu;
      hv[8 * q + 2 * i + 1] = xs.d[j][q][i] >> 16;
    }
}

// A pair of raw 16-bit activations of chunk j as one dword: element a in the low half,
// element b in the high half (a and b of the same parity), by one byte permute.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pair_raw(const XStage& xs, int j, int a, int b) {
  const uint32_t lo = xs.d[j][(a >> 1) >> 2][(a >> 1) & 3], hi = xs.d[j][(b >> 1) >> 2][(b >> 1) & 3];
  return __builtin_amdgcn_perm(hi, lo, (a & 1) ? 0x07060302u : 0x05040100u);
}

template <int XT>
__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return XT == XBF16 ? bf16_to_f32(h) : f16_to_f32(h);
}

template <int FMT, int XT, bool SIX>
__device__ void stage_compute(const MfmaArgs& A, int M, char* smem, const LdsLayout& L, int k0, int WK,
                              const XStage& xs) {
  using F = Fmt<FMT>;
  constexpr bool HAD = FMT == HAD2;
  constexpr bool NORM = x_rescaled(FMT, XT);
  constexpr bool BF = bf16_codes(FMT, XT);
  const int tid = threadIdx.x;
  const int nchunks = WK / 32;
  const int ntask = M * nchunks;
  const int pitch = A.a_pitch;
  float* rowf = reinterpret_cast<float*>(smem + L.row_off);  // [0..7] f, [8..15] 1/f
  uint32_t* rowmax = reinterpret_cast<uint32_t*>(smem + L.row_off);

  if constexpr (NORM) {
    if (tid < MAXM) rowmax[tid] = 0u;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      const int t = stage_task<SIX>(tid, j);
      if (t < ntask) {
        // magnitudes of one 16-bit float type order like their bit patterns with the sign
        // cleared: two per packed integer max
        u16x2 mx2 = {0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, xs.d[j][q][i] & 0x7FFF7FFFu));
        const uint32_t mb = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
        atomicMax(&rowmax[xs.m[j]], __float_as_uint(half_bits_to_f32<XT>(mb)));
      }
    }
    lds_barrier();
    if (tid < MAXM) {
      const float mx = __uint_as_float(rowmax[tid]);
      int ex = 0;
      float f = 1.0f;
      if (mx > 0.0f && mx == mx) {
        frexpf(mx, &ex);                      // mx < 2^ex
        int e = 14 - ex - (HAD ? 4 : 0);      // rotated values are below sqrt(256) * max = 16 * max
        e = e < -120 ? -120 : (e > 120 ? 120 : e);
        f = ldexpf(1.0f, e);
      }
      rowf[tid] = f;
      rowf[MAXM + tid] = 1.0f / f;
    }
    lds_barrier();
  }

#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    const int t = stage_task<SIX>(tid, j);
    if (t >= ntask) continue;   // whole blocks of 8 lanes skip together (32 | ntask, 64 | 6 * 64)
    const int m = xs.m[j], c = xs.c[j];
    uint32_t hv[32];  // rotated and rescaled fp16 bits, natural K order (rotated format only)
    float scale = 1.0f;
    if constexpr (NORM) scale = rowf[m];
    if constexpr (HAD) {
      chunk_halves(xs, j, hv);
      float v[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = half_bits_to_f32<XT>(hv[e]);
      if (A.signs) {
        const uint32_t sw = A.signs[(k0 >> 5) + c];   // the chunk's 32 sign bits
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((sw >> e) & 1u) << 31));
      }
      scale *= fwht_lanes(v, c & ((1 << A.had_stages) - 1), A.had_stages) * A.had_scale;
#pragma unroll
      for (int e = 0; e < 32; ++e) hv[e] = f32_to_f16_bits(v[e] * scale);
    }
    // Activations a (low half) and b (high half) of the chunk as an operand pair.  bf16
    // input against 2-bit codes: the power-of-two rescale maps it exactly into fp16 (8
    // significant bits fit in 11; only values over 2^27 times smaller than the row maximum
    // reach the fp16 subnormals), so converting a pair at once with truncation gives the
    // same halves.  Against 1-bit codes bf16 stays bf16 (the codes decode to bf16).
    auto pair = [&](int a, int b) -> uint32_t {
      if constexpr (HAD) {
        return hv[a] | (hv[b] << 16);
      } else if constexpr (NORM) {
        const uint32_t da = xs.d[j][(a >> 1) >> 2][(a >> 1) & 3], db = xs.d[j][(b >> 1) >> 2][(b >> 1) & 3];
        const float fa = __uint_as_float((a & 1) ? (da & 0xFFFF0000u) : (da << 16));
        const float fb = __uint_as_float((b & 1) ? (db & 0xFFFF0000u) : (db << 16));
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fa * scale, fb * scale));
      } else {
        return pair_raw(xs, j, a, b);
      }
    };

    // pair dwords, sums, LDS writes
    char* arow = smem + L.a_off + m * pitch;
    if constexpr (F::ONE_BIT) {
      // chunk = one word window (32 K) = word (c % 4) of group (c / 4).  The offset sum is
      // sum a (BETA + 1) for signs (the decoded half is BETA + 2 bit = BETA + 1 + sign) and
      // sum a BETA for 1-bit affine codes (BETA + 2 bit = BETA + 2 code).
      uint32_t pd[16];
      float e = 0.0f, xsum = 0.0f;
#pragma unroll
      for (int b0 = 0; b0 < 16; ++b0) {
        pd[b0] = pair(b0, b0 + 16);
        if constexpr (BF) {
          // BETA + 1 is no bf16 value beyond 128: sum a BETA and sum a apart
          const bf16x2 ph = __builtin_bit_cast(bf16x2, pd[b0]);
          const __bf16 cb = (__bf16)sign1_beta_bf16(b0), one = (__bf16)1.0f;
          e = __builtin_amdgcn_fdot2_f32_bf16(ph, bf16x2{cb, cb}, e, false);
          xsum = __builtin_amdgcn_fdot2_f32_bf16(ph, bf16x2{one, one}, xsum, false);
        } else {
          const _Float16 cf = (_Float16)(sign1_beta(b0) + (FMT == SIGN1 ? 1.0f : 0.0f));
          const f16x2 ph = __builtin_bit_cast(f16x2, pd[b0]);
          e = __builtin_amdgcn_fdot2(ph, f16x2{cf, cf}, e, false);
          if constexpr (F::AFFINE) xsum = __builtin_amdgcn_fdot2(ph, f16x2{(_Float16)1.0f, (_Float16)1.0f}, xsum, false);
        }
      }
      if constexpr (BF && FMT == SIGN1) e += xsum;
      u32x4* dst = reinterpret_cast<u32x4*>(arow + (c >> 2) * F::GS + (c & 3) * F::WB);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = u32x4{pd[4 * q], pd[4 * q + 1], pd[4 * q + 2], pd[4 * q + 3]};
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      if constexpr (F::AFFINE) {
        xsum += __shfl_xor(xsum, 1);
        xsum += __shfl_xor(xsum, 2);
      }
      if ((c & 3) == 0) {
        const int grp = c >> 2;
        reinterpret_cast<float*>(smem + L.e_off)[grp * MAXM + m] = -e;
        if constexpr (F::AFFINE && BF) {
          // group sum / 128 as bf16 hi and lo parts (unscaled bf16 rows can exceed fp16's
          // range): the quad of GL = 2 groups holds (hi, lo) twice, K slots
          // [hi0 hi1 lo0 lo1 hi0 hi1 lo0 lo1] against biases [bh bh bl bl] (compute_unit)
          const float xm = xsum * (1.0f / F::G);
          const uint32_t hb = __float_as_uint(xm) >> 16;
          const float lo = xm - __uint_as_float(hb << 16);   // exact
          const uint16_t lb = __builtin_bit_cast(uint16_t, (__bf16)lo);
          uint16_t* xp = reinterpret_cast<uint16_t*>(smem + L.xp_off + m * L.xp_pitch + (grp / F::GL) * 16);
          const int h = grp % F::GL;
          xp[h] = xp[4 + h] = (uint16_t)hb;
          xp[2 + h] = xp[6 + h] = lb;
        } else if constexpr (F::AFFINE) {
          // group sum / 128 as fp16 hi and lo parts; a quad holds GL = 2 groups, its unused
          // halves are cleared by the quad's first group
          const float xm = xsum * (1.0f / F::G);
          const _Float16 hi = (_Float16)xm;
          const _Float16 lo = (_Float16)(xm - (float)hi);
          _Float16* xp = reinterpret_cast<_Float16*>(smem + L.xp_off + m * L.xp_pitch + (grp / F::GL) * 16);
          xp[grp % F::GL] = hi;
          xp[4 + grp % F::GL] = lo;
          if (grp % F::GL == 0) {
            xp[2] = xp[3] = xp[6] = xp[7] = (_Float16)0.0f;
          }
        }
      }
    } else {
      // chunk = two word windows (16 K each) = words 2(c%2), 2(c%2)+1 of group c/2
      float r = 0.0f, xsum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 2; ++ww) {
        uint32_t pd[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          pd[jj] = pair(16 * ww + jj, 16 * ww + jj + 8);
          const _Float16 bj = (_Float16)affine2_beta(jj);
          const f16x2 ph = __builtin_bit_cast(f16x2, pd[jj]);
          r = __builtin_amdgcn_fdot2(ph, f16x2{bj, bj}, r, false);
          xsum = __builtin_amdgcn_fdot2(ph, f16x2{(_Float16)1.0f, (_Float16)1.0f}, xsum, false);
        }
        u32x4* dst = reinterpret_cast<u32x4*>(arow + (c >> 1) * F::GS + (2 * (c & 1) + ww) * F::WB);
        dst[0] = u32x4{pd[0], pd[1], pd[2], pd[3]};
        dst[1] = u32x4{pd[4], pd[5], pd[6], pd[7]};
      }
      r += __shfl_xor(r, 1);
      xsum += __shfl_xor(xsum, 1);
      if ((c & 1) == 0) {
        const int grp = c >> 1;
        reinterpret_cast<float*>(smem + L.e_off)[grp * MAXM + m] = -r;
        // the group sum enters the bias product as an exact-enough fp16 pair: X/64 is
        // bounded by the largest activation, so neither part can overflow
        const float xm = xsum * (1.0f / F::G);
        const _Float16 hi = (_Float16)xm;
        const _Float16 lo = (_Float16)(xm - (float)hi);
        _Float16* xp = reinterpret_cast<_Float16*>(smem + L.xp_off + m * L.xp_pitch + (grp / F::GL) * 16);
        xp[grp % F::GL] = hi;
        xp[4 + grp % F::GL] = lo;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Loaded data of one unit for one lane: GL consecutive 16-byte groups of the lane's row
// and their fp16 scales (and biases) as loaded.  From separate arrays, s and b hold
// scale pairs and bias pairs (group 2d in the low half of word d); from the interleaved
// layout (SBI), s holds the GL (scale, bias) words of the lane's groups, one 16-byte (or
// 8-byte) load, and b is unused.  Nothing consumes a load where it is issued, so the loads
// of later units stay in flight.
template <int FMT, bool SBI> struct Unit {
  u32x4 w[Fmt<FMT>::GL];
  uint32_t s[SBI ? Fmt<FMT>::GL : Fmt<FMT>::GL / 2];
  uint32_t b[Fmt<FMT>::GL / 2];
};

__device__ __forceinline__ float half_of(uint32_t pair, int hi) {
  return (float)__builtin_bit_cast(f16x2, pair)[hi];
}

// Code extraction with the masks and magics held in registers (one v_and_or_b32 per
// operand register; as literals the compiler would split it into an AND and an OR).
template <int FMT, bool BF>
__device__ __forceinline__ void unpack_word_rt(uint32_t w, uint32_t* out, const uint32_t* mk, const uint32_t* mg) {
  if constexpr (BF) {
    const uint32_t src[2] = {w, w >> 8};
#pragma unroll
    for (int b0 = 0; b0 < 16; ++b0) out[b0] = (src[b0 >> 3] & mk[b0 & 7]) | mg[b0 & 7];
  } else if constexpr (Fmt<FMT>::ONE_BIT) {
    const uint32_t src[3] = {w, w << 5, w >> 6};
#pragma unroll
    for (int b0 = 0; b0 < 16; ++b0) {
      const int k = sign1_pos(b0) - 5;
      out[b0] = (src[sign1_src(b0)] & mk[k]) | mg[k];
    }
  } else {
    const uint32_t src[3] = {w, w << 6, w >> 6};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = (affine2_pos(j) - 4) >> 1;
      out[j] = (src[affine2_src(j)] & mk[k]) | mg[k];
    }
  }
}

// One unit of one lane, as a pipeline over pairs of quantization groups.  The two groups
// of a pair run as two independent MFMA chains (each accumulator holds one group's dot
// products, so the group's scale applies once per accumulator); the A operands of the
// next step are read from LDS while the current step's words are decoded and multiplied.
//   Mode Q: lane-group g owns groups GL*g + h; pairs (h, h+1), 4 words each.
//   Mode H: lane-group pair p = g/2 shares groups (2p + u)*GL + h (u = 0, 1); pair = the
//           two groups u = 0, 1 at one h, 2 words each after a permlane16 swap of words.
//   a_lane: LDS address of the lane's operand window for its first group at this step
//   e_lane: LDS address of the offset sums of that group for the lane's accumulator rows
//   xp_lane: LDS address of the lane's quad of group sums (2-bit formats)
// The 2-bit bias term sum_g b_g X_g is one more MFMA per unit: A = (X/64 hi, X/64 lo) of
// the lane-group's GL groups, B = (b, b) of the same groups, accumulated into yb.
template <int FMT>
__device__ __forceinline__ void read_a(const char* smem, uint32_t addr, f16x8* dst) {
#pragma unroll
  for (int q = 0; q < Fmt<FMT>::NQ; ++q) dst[q] = *reinterpret_cast<const f16x8*>(smem + addr + 16 * q);
}

// AMASK: only the lanes whose operand row is a drafted row (a_on) read their A operands; the
// others keep the zeros abuf was cleared to.  abuf lives across units for that reason.
template <int FMT, int MODE, bool BF, bool AMASK, bool SBI>
__device__ __forceinline__ void compute_unit(const Unit<FMT, SBI>& U, const char* smem, uint32_t a_lane, uint32_t e_lane,
                                             uint32_t xp_lane, const uint32_t* mk, const uint32_t* mg,
                                             float yacc[4], f32x4& yb, bool a_on,
                                             f16x8 (&abuf)[2][2 * Fmt<FMT>::NQ]) {
  using F = Fmt<FMT>;
  constexpr int GL = F::GL, NQ = F::NQ;
  constexpr int NPAIR = MODE == VAR_MFMA_Q ? GL / 2 : GL;
  constexpr int WPP = MODE == VAR_MFMA_Q ? 4 : 2;   // words per group and pair member
  constexpr int NSTEP = NPAIR * WPP;
  // 1-bit affine codes decode to BETA + 2 code, so their accumulators hold twice the sum
  constexpr float SCALE_MUL = FMT == AFFINE1 ? 0.5f : 1.0f;
  // scale pairs and bias pairs of the lane's groups (group 2d in the low half of word d);
  // from interleaved (scale, bias) words, two byte permutes per pair
  uint32_t us[GL / 2], ub[GL / 2];
#pragma unroll
  for (int d = 0; d < GL / 2; ++d) {
    if constexpr (SBI) {
      us[d] = __builtin_amdgcn_perm(U.s[2 * d + 1], U.s[2 * d], 0x05040100u);
      ub[d] = __builtin_amdgcn_perm(U.s[2 * d + 1], U.s[2 * d], 0x07060302u);
    } else {
      us[d] = U.s[d];
      ub[d] = F::AFFINE ? U.b[d] : 0u;
    }
  }

  uint32_t wa[NPAIR][WPP], wb[NPAIR][WPP];
  float sa[NPAIR], sb[NPAIR];
  int ga[NPAIR], gb[NPAIR];   // unit-relative group slots (units of GS) of the pair
  if constexpr (MODE == VAR_MFMA_Q) {
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wa[pi][w] = U.w[2 * pi][w];
        wb[pi][w] = U.w[2 * pi + 1][w];
      }
      sa[pi] = half_of(us[pi], 0) * SCALE_MUL;
      sb[pi] = half_of(us[pi], 1) * SCALE_MUL;
      ga[pi] = 2 * pi;
      gb[pi] = 2 * pi + 1;
    }
  } else {
    // the swap of a register with itself hands lane-group pair p the scale pairs of both
    // lane-groups 2p ([0]) and 2p+1 ([1])
    uint32_t sc[2][GL / 2];
#pragma unroll
    for (int d = 0; d < GL / 2; ++d) {
      const auto t = __builtin_amdgcn_permlane16_swap(us[d], us[d], false, false);
      sc[0][d] = t[0];
      sc[1][d] = t[1];
    }
#pragma unroll
    for (int h = 0; h < GL; ++h) {
      // words 2,3 of the even lane-group trade places with words 0,1 of the odd one
      const auto s02 = __builtin_amdgcn_permlane16_swap(U.w[h][0], U.w[h][2], false, false);
      const auto s13 = __builtin_amdgcn_permlane16_swap(U.w[h][1], U.w[h][3], false, false);
      wa[h][0] = s02[0];
      wa[h][1] = s13[0];
      wb[h][0] = s02[1];
      wb[h][1] = s13[1];
      sa[h] = half_of(sc[0][h >> 1], h & 1) * SCALE_MUL;
      sb[h] = half_of(sc[1][h >> 1], h & 1) * SCALE_MUL;
      ga[h] = h;
      gb[h] = GL + h;
    }
  }

  if (!AMASK || a_on) {
    read_a<FMT>(smem, a_lane + ga[0] * F::GS, abuf[0]);
    read_a<FMT>(smem, a_lane + gb[0] * F::GS, abuf[0] + NQ);
  }
  f32x4 ea = *reinterpret_cast<const f32x4*>(smem + e_lane + ga[0] * (MAXM * 4));
  f32x4 eb = *reinterpret_cast<const f32x4*>(smem + e_lane + gb[0] * (MAXM * 4));
  f32x4 acc_a = ea, acc_b = eb;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int pi = st / WPP, w = st % WPP;
    if (st + 1 < NSTEP) {
      const int pn = (st + 1) / WPP, wn = (st + 1) % WPP;
      if (!AMASK || a_on) {
        read_a<FMT>(smem, a_lane + ga[pn] * F::GS + wn * F::WB, abuf[(st + 1) & 1]);
        read_a<FMT>(smem, a_lane + gb[pn] * F::GS + wn * F::WB, abuf[(st + 1) & 1] + NQ);
      }
    }
    if (w == 0) {
      acc_a = ea;
      acc_b = eb;
      if (pi + 1 < NPAIR) {   // the next pair's offset sums, one pair ahead
        ea = *reinterpret_cast<const f32x4*>(smem + e_lane + ga[pi + 1] * (MAXM * 4));
        eb = *reinterpret_cast<const f32x4*>(smem + e_lane + gb[pi + 1] * (MAXM * 4));
      }
    }
    uint32_t pa[F::PAIRS], pb[F::PAIRS];
    unpack_word_rt<FMT, BF>(wa[pi][w], pa, mk, mg);
    unpack_word_rt<FMT, BF>(wb[pi][w], pb, mk, mg);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const u32x4 ba = u32x4{pa[4 * q], pa[4 * q + 1], pa[4 * q + 2], pa[4 * q + 3]};
      const u32x4 bb = u32x4{pb[4 * q], pb[4 * q + 1], pb[4 * q + 2], pb[4 * q + 3]};
      if constexpr (BF) {
        acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, abuf[st & 1][q]),
                                                         __builtin_bit_cast(bf16x8, ba), acc_a, 0, 0, 0);
        acc_b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, abuf[st & 1][NQ + q]),
                                                         __builtin_bit_cast(bf16x8, bb), acc_b, 0, 0, 0);
      } else {
        acc_a = __builtin_amdgcn_mfma_f32_16x16x32_f16(abuf[st & 1][q], __builtin_bit_cast(f16x8, ba), acc_a, 0, 0, 0);
        acc_b = __builtin_amdgcn_mfma_f32_16x16x32_f16(abuf[st & 1][NQ + q], __builtin_bit_cast(f16x8, bb), acc_b, 0, 0, 0);
      }
    }
    if (w == WPP - 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(sa[pi], acc_a[r], __builtin_fmaf(sb[pi], acc_b[r], yacc[r]));
    }
  }
  if constexpr (F::AFFINE) {
    // K slots: the lane-group's GL group sums as hi parts (halves 0..3), then lo parts
    // (halves 4..7); with GL = 2 the unused halves are zero on both sides
    const f16x8 xa = *reinterpret_cast<const f16x8*>(smem + xp_lane);
    if constexpr (BF) {
      // bf16 (X hi, X lo) against the two fp16 biases split exactly into bf16 hi + lo
      // (11 significant bits = 8 + 3): every cross product of the parts is one K slot
      static_assert(GL == 2, "bf16 bias quads hold two groups");
      const float f0 = half_of(ub[0], 0), f1 = half_of(ub[0], 1);
      const float l0 = f0 - __uint_as_float(__float_as_uint(f0) & 0xFFFF0000u);
      const float l1 = f1 - __uint_as_float(__float_as_uint(f1) & 0xFFFF0000u);
      const uint32_t dh = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      const uint32_t dl = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
      yb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                   __builtin_bit_cast(bf16x8, u32x4{dh, dh, dl, dl}), yb, 0, 0, 0);
    } else {
      u32x4 bw;
      if constexpr (GL == 4) bw = u32x4{ub[0], ub[1], ub[0], ub[1]};
      else bw = u32x4{ub[0], 0u, ub[0], 0u};
      yb = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, __builtin_bit_cast(f16x8, bw), yb, 0, 0, 0);
    }
  } else {
    (void)xp_lane;
    (void)yb;
  }
}

// Debug decode of packed codes through the GEMM's own register extraction:
// unpack_word_rt with the masks and magics decode_consts builds for the call's format and
// activation dtype.  Every operand half holds BETA + DELTA * code, so the code is
// (half - BETA) / DELTA, written as one byte per weight; a half that is not exactly
// BETA + DELTA * c for a code c in range gives 0xFF, which no code equals.  Register j
// holds the codes at K offsets j and j + WORD_K / 2 of its word.
struct DecodeArgs {
  const uint32_t* w;
  uint8_t* codes;
  int N, K;
  uint32_t mask[8], magic[8];
};

template <int FMT, bool BF>
__global__ __launch_bounds__(256) void vg_debug_decode(DecodeArgs D) {
  using F = Fmt<FMT>;
  constexpr int WK = F::WORD_K, NREG = F::PAIRS;
  constexpr float DELTA = F::ONE_BIT ? SIGN1_DELTA : AFFINE2_DELTA;
  constexpr int CMAX = F::ONE_BIT ? 1 : 3;
  const size_t wpr = (size_t)(D.K / WK);
  const size_t gw = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gw >= (size_t)D.N * wpr) return;
  const size_t n = gw / wpr, wi = gw - n * wpr;
  uint32_t mk[8], mg[8], r[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    mk[k] = D.mask[k];
    mg[k] = D.magic[k];
  }
  unpack_word_rt<FMT, BF>(D.w[gw], r, mk, mg);
  uint8_t* out = D.codes + n * (size_t)D.K + (size_t)WK * wi;
#pragma unroll
  for (int j = 0; j < NREG; ++j) {
    const float beta = BF ? sign1_beta_bf16(j) : (F::ONE_BIT ? sign1_beta(j) : affine2_beta(j));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t bits = h ? r[j] >> 16 : r[j] & 0xFFFFu;
      const float c = ((BF ? bf16_to_f32(bits) : f16_to_f32(bits)) - beta) / DELTA;
      const int ci = (int)c;
      out[j + h * (WK / 2)] = ((float)ci == c && ci >= 0 && ci <= CMAX) ? (uint8_t)ci : (uint8_t)0xFF;
    }
  }
}

// Finishes a wave's contribution to tile t for the current window: undo the row scaling,
// sum the lane-groups holding the same rows (register swaps between lane rows), then
// either add into the tile accumulator (sole contributor; the first window stores, so the
// accumulator needs no clearing) or park it in the wave's slot for the fixed-order
// reduction.
template <int FMT, int MODE>
__device__ __forceinline__ void flush_tile(char* smem, const LdsLayout& L, int t, bool sole, bool first, int slot,
                                           int wid, int g, int i, const float yacc[4], const f32x4& yb) {
  const float* invf = reinterpret_cast<const float*>(smem + L.row_off) + MAXM;
  const int m0 = MODE == VAR_MFMA_Q ? 0 : 4 * (g & 1);
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = (Fmt<FMT>::AFFINE ? __builtin_fmaf((float)Fmt<FMT>::G, yb[r], yacc[r]) : yacc[r]) * invf[m0 + r];
    if constexpr (MODE == VAR_MFMA_Q) {
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[r]), __float_as_uint(v[r]), false, false);
      v[r] = __uint_as_float(p[0]) + __uint_as_float(p[1]);   // rows 0+1 and 2+3
    }
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[r]), __float_as_uint(v[r]), false, false);
    v[r] = __uint_as_float(h[0]) + __uint_as_float(h[1]);     // lanes l and l^32
  }
  const bool writer = MODE == VAR_MFMA_Q ? (g == 0) : (g < 2);
  if (writer) {
    float* dst = sole ? reinterpret_cast<float*>(smem + L.ytile_off) + t * (MAXM * 16)
                      : reinterpret_cast<float*>(smem + L.slot_off) + (wid * 2 + slot) * (MAXM * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* p = dst + (m0 + r) * 16 + i;
      *p = sole && !first ? *p + v[r] : v[r];
    }
  }
}

// Grouped expert verify: this workgroup's job, derived from the routing by every workgroup
// alike.  Entry l = m * topk + s (row m, slot s) is routed to expert route[l] when that is
// in 0..E-1.  Each expert's entries, in order of l, fill jobs of at most cap rows; jobs
// are numbered by expert, then by position.  With J jobs each takes rg = max(rg_min,
// grid / J) row groups (at most one per 16-row tile), and workgroup b takes row group
// b % rg of job b / rg (J * rg <= grid: the grid holds rg_min row groups of the most jobs
// a routing can make).  The job's x rows (job[0..7]), y rows (job[8..15]), J (job[16]),
// expert (job[17]) and row count (job[18]) are left in LDS; the 64-entry scratch after
// them lies in the activation area, which is written only after the last barrier here.
// Returns false when the workgroup has no job.
__device__ bool find_job(const MfmaArgs& A, char* smem, int& M, int& expert, int& rgi, int& rg) {
  int* job = reinterpret_cast<int*>(smem);
  int* key = job + JOB_BYTES / 4;   // [64] expert of each entry, -1 when unused
  int* starts = key + 64;           // [64] jobs begun by each expert's first entry
  const int tid = threadIdx.x;
  const int n = A.M * A.topk, cap = A.cap;
  if (tid < 64) {
    const int v = tid < n ? A.route[tid] : -1;
    key[tid] = (v >= 0 && v < A.E) ? v : -1;
  }
  lds_barrier();
  int e = -1, pos = 0, cnt = 0;
  if (tid < 64) {
    e = key[tid];
#pragma unroll 8
    for (int t = 0; t < 64; ++t) {
      const int kt = key[t];
      cnt += kt == e ? 1 : 0;
      pos += (kt == e && t < tid) ? 1 : 0;
    }
    starts[tid] = (e >= 0 && pos == 0) ? (cnt + cap - 1) / cap : 0;
  }
  lds_barrier();
  const int tiles = (A.N + 15) / 16;
  if (tid < 64) {
    int before = 0, total = 0;
#pragma unroll 8
    for (int t = 0; t < 64; ++t) {
      const int jt = starts[t];
      total += jt;
      before += key[t] < e ? jt : 0;
    }
    if (tid == 0) job[16] = total;
    if (e >= 0 && total > 0) {
      const int r_dyn = min(tiles, max(A.rg, (int)gridDim.x / total));
      const int mine = before + pos / cap, r = pos - (pos / cap) * cap;
      if (mine == (int)blockIdx.x / r_dyn) {
        job[r] = tid / A.topk;
        job[MAXM + r] = tid;
        if (r == 0) {
          job[17] = e;
          job[18] = min(cap, cnt - pos);
        }
      }
    }
  }
  lds_barrier();
  const int total = job[16];
  if (total == 0) return false;
  rg = min(tiles, max(A.rg, (int)gridDim.x / total));
  const int j = (int)blockIdx.x / rg;
  if (j >= total) return false;
  rgi = (int)blockIdx.x - j * rg;
  expert = job[17];
  M = job[18];
  return true;
}

// Fused argmax of the output head (the head's verify is checked by its argmax): each
// (value, column) of a row becomes one 64-bit key that orders like (value, -column) --
// larger value first, then the lower column -- and NaN never enters.  A workgroup leaves its
// largest key of each row in its own slot of amax_key (row m at amax_key[FUSED_KEYS *
// blockIdx.x + m], zero for a row with no key), with plain stores: no counter and no wait,
// and a one-workgroup kernel after the GEMM (launch_argmax_keys) picks each row's winner.
__device__ __forceinline__ unsigned long long arg_key(float v, int n) {
  const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);   // -0 ties with +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // orders like v
  return ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)n;
}

static_assert(FUSED_KEYS == MAXM, "a workgroup keeps one key slot per row");
// After the barrier finish: wave m takes row m of the workgroup's columns from ytile.
__device__ void fused_argmax(const MfmaArgs& A, const float* ytile, int M, int r0, int nr, int wid, int lane) {
  if (wid >= M) return;
  unsigned long long best = 0ull;
  for (int rr = lane; rr < nr; rr += 64) {
    const float v = ytile[(rr >> 4) * (MAXM * 16) + wid * 16 + (rr & 15)];
    if (v == v) {
      const unsigned long long k = arg_key(v, r0 + rr);
      best = k > best ? k : best;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if (lane == 0) A.amax_key[(size_t)blockIdx.x * FUSED_KEYS + wid] = best;
}

template <int FMT, int MODE, int XT, int PREF, bool AMASK, bool EARLY, bool SBI, bool DIRECT, bool SIX, bool DARG>
__device__ __forceinline__ void mfma_body(const MfmaArgs& A, char* smem) {
  static_assert(DIRECT || !DARG, "the argmax of the direct finish needs the direct finish");
  using F = Fmt<FMT>;
  constexpr int GL = F::GL, GPS = 4 * GL;
  constexpr bool NORM = x_rescaled(FMT, XT);
  constexpr bool BF = bf16_codes(FMT, XT);
  constexpr int NMK = BF ? 8 : 6;   // bit positions in use
  // The workgroup's job: row group and K slice of the call, or for a grouped expert verify
  // a row group of one job, whose rows are gathered from x and scattered to y.
  int M = A.M, rgi, ksi = 0, rg = A.rg;
  const uint32_t* wq = A.w;
  const uint16_t* sc = A.scales;
  const uint16_t* bi = A.biases;
  const int* xmap = nullptr;   // grouped: x row of each row, then y row of each row
  if (A.route) {
    int e;
    if (!find_job(A, smem, M, e, rgi, rg)) return;
    xmap = reinterpret_cast<const int*>(smem);
    wq = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(wq) + e * A.w_estride);
    sc = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(sc) + e * A.s_estride);
    if (bi) bi = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(bi) + e * A.s_estride);
  } else {
    rgi = A.ks == 1 ? (int)blockIdx.x : (int)__umulhi(blockIdx.x, A.ks_magic);
    ksi = blockIdx.x - rgi * A.ks;
  }
  const LdsLayout L = A.route ? LdsLayout(FMT, M, A.win_steps, A.tiles_max) : A.lay;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  // row group rgi: rows [r0, r1), the first N % rg groups one row longer
  const int rq = A.route ? A.N / rg : A.rq, rrem = A.route ? A.N - rq * rg : A.rrem;
  const int r0 = rgi * rq + min(rgi, rrem), r1 = r0 + rq + (rgi < rrem ? 1 : 0);
  const int T = (r1 - r0 + 15) / 16;
  const int S = A.K / KSTEP;
  // this slice's K-steps, S * ksi / ks and S * (ksi + 1) / ks
  const int kb0 = A.ks == 1 ? 0 : (int)__umulhi((uint32_t)(S * ksi), A.ks_magic);
  const int kb1 = A.ks == 1 ? S : (int)__umulhi((uint32_t)(S * (ksi + 1)), A.ks_magic);
  const uint32_t wrow = (uint32_t)(A.K / F::WORD_K) * 4u;   // bytes of codes per row
  const uint32_t srow = (uint32_t)(A.K / F::G) * 2u;        // bytes of scales per row
  // masks stay in SGPRs, magics are moved into VGPRs once: v_and_or_b32 may read only one
  // scalar operand, and with both scalar the compiler would emit a separate AND and OR.
  uint32_t mk[NMK], mg[NMK];
#pragma unroll
  for (int k = 0; k < NMK; ++k) {
    mk[k] = A.mask[k];
    asm volatile("v_mov_b32 %0, %1" : "=v"(mg[k]) : "s"(A.magic[k]));
  }

  // this lane's operand row: a drafted row, or the zero row M when the lane's A row
  // carries none (rows of other row-blocks must read zeros in this lane's K slots)
  const int am = MODE == VAR_MFMA_Q ? i - 4 * g : (g < 2 ? i : i - 8);
  const bool av = am >= 0 && am < M && (MODE == VAR_MFMA_H || am < 4);
  const int m0 = MODE == VAR_MFMA_Q ? 0 : 4 * (g & 1);
  // The lanes without a drafted row all read one address of the zero row, whatever their
  // lane-group: a single extra distinct address per LDS read instead of one per lane-group
  // (a 128-bit read takes as many passes as the most distinct addresses any 16-byte bank
  // slot of 128 bytes holds; at 8 rows the real rows fill every slot four deep, and four
  // zero-row addresses made two slots six deep).
  const uint32_t a_lane0 = av ? L.a_off + (uint32_t)am * A.a_pitch +
                                    (MODE == VAR_MFMA_Q ? GL * g * F::GS : 2 * (g >> 1) * GL * F::GS + 2 * (g & 1) * F::WB)
                              : L.a_off + (uint32_t)M * A.a_pitch;
  const uint32_t e_lane0 = L.e_off + ((MODE == VAR_MFMA_Q ? GL * g : 2 * (g >> 1) * GL) * MAXM + m0) * 4;
  const uint32_t xp_lane0 = av ? L.xp_off + (uint32_t)am * L.xp_pitch + (uint32_t)g * 16u
                               : L.xp_off + (uint32_t)M * L.xp_pitch;

  f16x8 abuf[2][2 * F::NQ];   // A operands, double-buffered across steps (see compute_unit)
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int q = 0; q < 2 * F::NQ; ++q) abuf[u][q] = f16x8{};
  float* ytile = reinterpret_cast<float*>(smem + L.ytile_off);
  {
    // the zero rows: never written by the staging, so cleared once per launch
    uint32_t* za = reinterpret_cast<uint32_t*>(smem + L.a_off + M * A.a_pitch);
    for (int e = tid; e < A.a_pitch / 16; e += NTHREADS) reinterpret_cast<u32x4*>(za)[e] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (F::AFFINE) {
      uint32_t* zx = reinterpret_cast<uint32_t*>(smem + L.xp_off + M * L.xp_pitch);
      for (int e = tid; e < L.xp_pitch / 16; e += NTHREADS) reinterpret_cast<u32x4*>(zx)[e] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if (!NORM && tid < MAXM) reinterpret_cast<float*>(smem + L.row_off)[MAXM + tid] = 1.0f;
  // One window over the slice's whole K, no K split, no argmax and no grouped job: every tile
  // goes to y from the wave that completes it, with no barrier after the loop.  A tile that
  // waves share is summed (in wave order, as below) by the last of them to arrive, counted in
  // the first word of the tile's accumulator, which such a tile leaves unused.
  if constexpr (DIRECT)
    for (int t = tid; t < T; t += NTHREADS) reinterpret_cast<uint32_t*>(ytile)[t * (MAXM * 16)] = 0u;
  // direct argmax: each row's largest key over the tiles stored so far (the split-tile
  // records' area, unused by the direct finish), and the waves done (the flag word)
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(smem + L.red_off);
  uint32_t* waves_done = reinterpret_cast<uint32_t*>(smem + L.flag_off);
  if constexpr (DARG) {
    if (tid < MAXM) keys[tid] = 0ull;
    if (tid == 0) waves_done[0] = 0u;
  }
  // direct argmax: the key of element v of row m at column col (none when ok is false) joins
  // the row's LDS maximum, each lane on its own: an LDS atomic whose result no one waits
  // for.  A cross-lane maximum first would chain several LDS permutes per tile, and a
  // running maximum per lane in registers measured no faster.
  auto note_key = [&](float v, bool ok, int m, int col) {
    if (ok && v == v) __hip_atomic_fetch_max(keys + m, arg_key(v, col), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };


  const char* wbase = reinterpret_cast<const char*>(wq) + (size_t)r0 * wrow;
  // interleaved (scale, bias) words: twice the bytes of the scales alone at every offset
  const char* sbase = reinterpret_cast<const char*>(sc) + (size_t)r0 * srow * (SBI ? 2 : 1);
  const char* bbase = reinterpret_cast<const char*>(bi) + (size_t)r0 * srow;

  for (int ws0 = kb0; ws0 < kb1; ws0 += A.win_steps) {
    const int ns = min(A.win_steps, kb1 - ws0);
    const int UW = T * ns;
    const int ua = (int)(((uint32_t)UW * wid) / NW), ub = (int)(((uint32_t)UW * (wid + 1)) / NW);
    const int nu = ub - ua;

    // Load cursor (tile lt, step ls), kept uniform; the lane part of a load address is a
    // per-tile constant, the rest is a scalar offset.  Each of the wave's units is loaded
    // once, PREF units ahead of the one computing.
    // ua / ns: a multiply-high for full windows (ua * ns < 2^27 here)
    const int ua_t = ns == 1 ? ua : (ns == A.win_steps ? (int)__umulhi((uint32_t)ua, A.ws_magic) : ua / ns);
    int lt = nu > 0 ? ua_t : 0, ls = nu > 0 ? ua - lt * ns : 0, issued = 0;
    uint32_t lw_lane = 0, ls_lane = 0;
    auto set_load_tile = [&](int t) {
      const int rr = min(16 * t + i, r1 - 1 - r0) - 16 * t;   // clamp rows past the range
      // 24-bit products (rr < 16, row pitches below 2^24): a plain 32-bit multiply-add.  As a
      // 32-bit product the compiler forms a 64-bit multiply-add whose unused high addend may
      // be given the register of a load still in flight, and then waits for that load.
      lw_lane = __umul24((uint32_t)rr, wrow) + (uint32_t)(g * GL) * 16u;
      ls_lane = __umul24((uint32_t)rr, srow) + (uint32_t)(g * GL) * 2u;
    };
    set_load_tile(lt);
    auto issue = [&](Unit<FMT, SBI>& U) {
      const size_t tw = (size_t)(16 * lt) * wrow + (size_t)(ws0 + ls) * (GPS * 16);
      const size_t ts = (size_t)(16 * lt) * srow + (size_t)(ws0 + ls) * (GPS * 2);
      const char* wp = wbase + tw + lw_lane;
#pragma unroll
      for (int h = 0; h < GL; ++h) U.w[h] = *reinterpret_cast<const u32x4*>(wp + 16 * h);
      if constexpr (SBI) {
        const char* mp = sbase + 2 * (ts + ls_lane);
        if constexpr (GL == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(mp);
#pragma unroll
          for (int j = 0; j < 4; ++j) U.s[j] = v[j];
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(mp);
          U.s[0] = v.x;
          U.s[1] = v.y;
        }
      } else if constexpr (GL == 2) {
        U.s[0] = *reinterpret_cast<const uint32_t*>(sbase + ts + ls_lane);
        if constexpr (F::AFFINE) U.b[0] = *reinterpret_cast<const uint32_t*>(bbase + ts + ls_lane);
      } else {
        const uint2 sv = *reinterpret_cast<const uint2*>(sbase + ts + ls_lane);
        U.s[0] = sv.x;
        U.s[1] = sv.y;
        if constexpr (F::AFFINE) {
          const uint2 bv = *reinterpret_cast<const uint2*>(bbase + ts + ls_lane);
          U.b[0] = bv.x;
          U.b[1] = bv.y;
        }
      }
      if (issued + 1 < nu) {
        ++issued;
        if (++ls == ns) { ls = 0; ++lt; set_load_tile(lt); }
      }
    };

    // The activation loads go first: loads leave a CU in order, so weight loads ahead of
    // them would hold back the staging (and every MFMA after it) by the whole burst, and
    // weight loads issued while the activations are still in flight delay them in the
    // memory system just as much.  With EARLY a wave issues its first PREF units once its
    // own activation data has landed, so their latency overlaps the staging arithmetic and
    // the barrier after it; without, after the staging.
    XStage xs;
    stage_load<XT, SIX>(A, M, xmap, ws0 * KSTEP, ns * KSTEP, xs);
    Unit<FMT, SBI> ring[PREF];
    lds_barrier();  // previous window's readers are done with the LDS
    if constexpr (EARLY) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's activations
#pragma unroll
      for (int d = 0; d < PREF; ++d)
        if (DIRECT || d < nu) issue(ring[d]);
    }
    // The tiles split between waves in this window, for the reduction after it: wave
    // boundary bw (lanes 0..NW-2 of wave 0) records, when it falls strictly inside a tile
    // and is that tile's first such boundary, the tile (first word, bit 31 marking a
    // record), the waves whose unit range meets it (mask, low half of the second word)
    // and which of them started before it (their slot 1; high half).  Written after the
    // barrier that ends the previous window's reduction, read after the one that follows
    // the staging.  (Not the last wave: it carries the extra unit when the units do not
    // divide evenly, and delaying its first load costs the whole call up to a
    // microsecond, measured on MI355X.)
    if (!DIRECT && wid == 0 && lane < NW - 1) {
      const int bw = lane + 1;
      const int B = (int)(((uint32_t)UW * bw) / NW);
      const int t = B / ns, t0 = t * ns;
      uint32_t rec = 0, who = 0;
      if (B > 0 && B < UW && B != t0 && !(bw > 1 && (int)(((uint32_t)UW * (bw - 1)) / NW) > t0)) {
        uint32_t mask = 0, late = 0;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          const int a2 = (int)(((uint32_t)UW * w2) / NW), b2 = (int)(((uint32_t)UW * (w2 + 1)) / NW);
          if (a2 < b2 && b2 > t0 && a2 < t0 + ns) {
            mask |= 1u << w2;
            if (a2 < t0) late |= 1u << w2;
          }
        }
        rec = (1u << 31) | (uint32_t)t;
        who = (late << 16) | mask;
      }
      reinterpret_cast<uint32_t*>(smem + L.red_off)[2 * lane] = rec;
      reinterpret_cast<uint32_t*>(smem + L.red_off)[2 * lane + 1] = who;
    }
    stage_compute<FMT, XT, SIX>(A, M, smem, L, ws0 * KSTEP, ns * KSTEP, xs);
    if constexpr (!EARLY) {
#pragma unroll
      for (int d = 0; d < PREF; ++d)
        if (DIRECT || d < nu) issue(ring[d]);
    }
    lds_barrier();

    // The waves carrying one unit more than the others finish last; giving them issue
    // priority on their SIMD shortens the window's slowest wave (measured on MI355X).
    if (nu > (int)((uint32_t)UW / NW)) __builtin_amdgcn_s_setprio(3);
    else __builtin_amdgcn_s_setprio(1);
    int ct = nu > 0 ? ua_t : 0, cs = nu > 0 ? ua - ct * ns : 0;
    float yacc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 yb = {0.f, 0.f, 0.f, 0.f};
    // direct: a shared tile's sum over its waves' slots, in wave order (non-waves add +0),
    // stored to y; element e of a tile is (row e / 16, column e % 16)
    auto reduce_store = [&](int t) {
      const float* slots = reinterpret_cast<const float*>(smem + L.slot_off);
      // the waves whose unit range meets the tile (mask) and which of them began before it
      // (late: their part sits in slot 1)
      const int t0 = t * ns;
      uint32_t mask = 0, late = 0;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const int a2 = (int)(((uint32_t)UW * w2) / NW), b2 = (int)(((uint32_t)UW * (w2 + 1)) / NW);
        if (a2 < b2 && b2 > t0 && a2 < t0 + ns) {
          mask |= 1u << w2;
          if (a2 < t0) late |= 1u << w2;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && M <= 4) break;
        const int e = lane + 64 * h, m = e >> 4, rr = 16 * t + (e & 15);
        float v[NW];
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) v[w2] = slots[(w2 * 2 + ((late >> w2) & 1u)) * (MAXM * 16) + e];
        float sum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) sum += ((mask >> w2) & 1u) ? v[w2] : 0.0f;
        const bool ok = m < M && rr < r1 - r0;
        if (ok) A.y[(size_t)m * A.N + r0 + rr] = sum;
        if constexpr (DARG) note_key(sum, ok, m, r0 + rr);
      }
    };
    int red_t = -1;   // direct: a shared tile this wave completed last, summed after the next issue
    for (int base = 0; base < nu; base += PREF) {
#pragma unroll
      for (int d = 0; d < PREF; ++d) {
        if (base + d < nu) {
          const uint32_t a_lane = a_lane0 + (uint32_t)cs * (GPS * F::GS);
          const uint32_t e_lane = e_lane0 + (uint32_t)cs * (GPS * MAXM * 4);
          const uint32_t xp_lane = xp_lane0 + (uint32_t)cs * 64u;   // 4 quads of groups per unit
          compute_unit<FMT, MODE, BF, AMASK, SBI>(ring[d], smem, a_lane, e_lane, xp_lane, mk, mg, yacc, yb, av, abuf);
          if (++cs == ns || base + d + 1 == nu) {
            const bool sole = ua <= ct * ns && ub >= (ct + 1) * ns;
            flush_tile<FMT, MODE>(smem, L, ct, sole, ws0 == kb0, ua >= ct * ns ? 0 : 1, wid, g, i, yacc, yb);
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[r] = 0.f;
            yb = f32x4{0.f, 0.f, 0.f, 0.f};
            if (DIRECT && !sole) {
              // count this wave's units of the shared tile in (its slot written first); the
              // wave that brings the count to the tile's ns units is the last to arrive
              const uint32_t cnt = (uint32_t)(min(ub, (ct + 1) * ns) - max(ua, ct * ns));
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
              uint32_t before = 0;
              if (lane == 0)
                before = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(ytile) + ct * (MAXM * 16), cnt,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              if (__builtin_amdgcn_readfirstlane(before) + cnt == (uint32_t)ns) red_t = ct;
            }
            cs = 0;
            ++ct;
          }
        }
        // refill the slot only while units remain: a load past the last unit would still
        // be in flight after the loop, and the first reuse of its registers would wait
        // for it.  Otherwise the slot is dead; saying so lets mode H's lane swaps work on
        // its registers in place instead of on copies.
        if (base + d + PREF < nu) issue(ring[d]);
        else ring[d] = Unit<FMT, SBI>{};
        if (DIRECT && red_t >= 0) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
          reduce_store(red_t);
          red_t = -1;
        }
      }
    }
    if constexpr (DIRECT) {
      // the tiles this wave holds alone, read back from its own accumulator writes
      for (int t = ua_t; nu > 0 && t * ns < ub; ++t) {
        if (ua > t * ns || ub < (t + 1) * ns) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && M <= 4) break;
          const int e = lane + 64 * h, m = e >> 4, rr = 16 * t + (e & 15);
          const bool ok = m < M && rr < r1 - r0;
          const float v = ytile[t * (MAXM * 16) + e];
          if (ok) A.y[(size_t)m * A.N + r0 + rr] = v;
          if constexpr (DARG) note_key(v, ok, m, r0 + rr);
        }
      }
      if constexpr (DARG) {
        // the last of the workgroup's waves to finish stores the rows' keys
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        uint32_t before = 0;
        if (lane == 0)
          before = __hip_atomic_fetch_add(waves_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(before) == (uint32_t)(NW - 1)) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
          if (lane < M) A.amax_key[(size_t)blockIdx.x * FUSED_KEYS + lane] = keys[lane];
        }
      }
      return;
    }
    lds_barrier();

    // fixed-order reduction of tiles split between waves: a tile is split when a wave
    // boundary falls strictly inside it; its contributors are the non-empty waves whose
    // unit range meets it, summed in wave order (a contributor's slot 0 holds the tile
    // its range starts in, slot 1 the tile it ends in).  Wave w takes boundary w + 1, two
    // elements per lane, so the boundaries reduce side by side (two per 128-thread group
    // in turn measured 0.1-0.3 us slower on MI355X); every wave's candidate slot is read at
    // once and non-contributors add +0.
    {
      const float* slots = reinterpret_cast<const float*>(smem + L.slot_off);
      const uint32_t* red = reinterpret_cast<const uint32_t*>(smem + L.red_off);
      const int bw = wid + 1;
      const uint32_t rec = bw < NW ? __builtin_amdgcn_readfirstlane(red[2 * (bw - 1)]) : 0u;
      if (rec >> 31) {
        const uint32_t who = __builtin_amdgcn_readfirstlane(red[2 * (bw - 1) + 1]);
        const int t = (int)(rec & 0x7FFFFFFFu);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = lane + 64 * h;           // element (row, col) of a tile
          float v[NW];
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) v[w2] = slots[(w2 * 2 + ((who >> (16 + w2)) & 1u)) * (MAXM * 16) + e];
          float sum = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) sum += ((who >> w2) & 1u) ? v[w2] : 0.0f;
          float* yt = ytile + t * (MAXM * 16) + e;
          *yt = ws0 == kb0 ? sum : *yt + sum;
        }
      }
    }
  }
  lds_barrier();

  // write y[m, r0 .. r1) from the tile accumulators; element e is (m, rr) with m = e / nr,
  // taken by a float reciprocal: (e + 1/2) / nr lies at least 1/(2 nr) from an integer,
  // beyond the product's rounding (at most 2^-20 for e < 8 nr) while nr < 2^19; the plan
  // keeps row ranges within 2^18 (an integer division per element measured 0.06 us slower
  // at 8 rows on MI355X)
  const int nr = r1 - r0;
  const float inv_nr = 1.0f / (float)nr;
  auto row_of = [&](int e) { return (int)(((float)e + 0.5f) * inv_nr); };
  if (A.ks == 1) {
    for (int e = tid; e < M * nr; e += NTHREADS) {
      const int m = row_of(e), rr = e - m * nr;
      A.y[(size_t)(xmap ? xmap[MAXM + m] : m) * A.N + r0 + rr] = ytile[(rr >> 4) * (MAXM * 16) + m * 16 + (rr & 15)];
    }
    if (A.idx) fused_argmax(A, ytile, M, r0, nr, wid, lane);
    return;
  }
  // K split across workgroups: park this slice's partial, and let the last slice of the row
  // group to arrive add all slices in slice order (the same order whichever arrives last).
  // The partials and the arrival counter are agent-scope atomic accesses, which bypass the
  // per-XCD L2 caches; a device-wide fence would instead write back and invalidate the
  // whole L2 of the XCD under every other workgroup running there.
  float* part = A.part + (size_t)ksi * M * A.N;
  for (int e = tid; e < M * nr; e += NTHREADS) {
    const int m = row_of(e), rr = e - m * nr;
    __hip_atomic_store(part + (size_t)m * A.N + r0 + rr, ytile[(rr >> 4) * (MAXM * 16) + m * 16 + (rr & 15)],
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partials have landed
  lds_barrier();
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem + L.flag_off);
  if (tid == 0) {
    const uint32_t before = __hip_atomic_fetch_add(A.counters + rgi * SPLIT_CTR_STRIDE, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = before == (uint32_t)(A.ks - 1) ? 1u : 0u;
  }
  lds_barrier();
  if (flag[0] == 0u) return;
  for (int e = tid; e < M * nr; e += NTHREADS) {
    const int m = row_of(e), rr = e - m * nr;
    const float* src = A.part + (size_t)m * A.N + r0 + rr;
    float sum = 0.0f;
    // up to 8 slices' loads in flight at once (each is a trip past the L2), added in slice
    // order
    for (int k0 = 0; k0 < A.ks; k0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[k] = k0 + k < A.ks ? __hip_atomic_load(src + (size_t)(k0 + k) * M * A.N, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k0 + k < A.ks) sum += v[k];
    }
    A.y[(size_t)m * A.N + r0 + rr] = sum;
  }
  if (tid == 0) __hip_atomic_store(A.counters + rgi * SPLIT_CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------
// vg_gemv: the verify GEMM on the vector ALUs for one or two rows, with the activations
// held in registers.  Wave w of a workgroup owns K-step w (1024 columns); lane (rho, gam)
// owns the 64 columns gam*64.. of that step and output row rho of each 4-row block, so a
// wave's load instruction reads 4 rows x 256 contiguous bytes (2-bit) or 4 x 128 (1-bit)
// and every lane multiplies its own 64 activations, loaded once per call and kept in
// registers as the operand pairs the register decode produces (no activation staging
// through LDS).  Each lane also forms its own offset sum (sum of a * BETA, plus the group
// sum for affine codes) from those registers.  Products are v_dot2 into fp32 (fp16, or
// bf16 for 1-bit codes against bf16 rows); bf16 rows against 2-bit codes and rotated rows
// are scaled by a power of two per row into fp16 as in the MFMA kernels (the row maximum
// over the whole K comes from all waves of the workgroup), and the rotation runs in
// registers (a 64-point transform per lane, then lane pairs for blocks of 128 and 256).
// The 16 lanes of a row are added in a fixed order (DPP within the row), and the K-steps'
// partials of a row through LDS in step order, so results do not depend on timing.
constexpr int GV_RPW = 4;     // output rows per wave instruction (16 lanes each)
constexpr int GV_MAXS = 16;   // K-steps (waves) per workgroup: K <= 16384

template <int CTRL>
__device__ __forceinline__ float gv_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int FMT, int XT, int MM, int PREF, bool SBI>
__global__ __launch_bounds__(GV_MAXS * 64) void vg_gemv(MfmaArgs A) {
  using F = Fmt<FMT>;
  constexpr bool ONE = F::ONE_BIT;
  constexpr bool HAD = FMT == HAD2;
  constexpr bool NORM = x_rescaled(FMT, XT);
  constexpr bool BF = bf16_codes(FMT, XT);
  constexpr int NMK = BF ? 8 : 6;
  constexpr int NWORD = ONE ? 2 : 4;      // code words per lane and unit (64 codes)
  constexpr int HALF = F::WORD_K / 2;     // operand pairs per word
  constexpr float SCALE_MUL = FMT == AFFINE1 ? 0.5f : 1.0f;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* rowmax = reinterpret_cast<float*>(smem);          // [MAXM]
  float* part = reinterpret_cast<float*>(smem) + 2 * MAXM; // [blocks][4][S][MM]
  const int tid = threadIdx.x, lane = tid & 63;
  const int st = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = (int)(blockDim.x >> 6);
  const int rho = lane >> 4, gam = lane & 15;
  const int kl = st * KSTEP + gam * 64;   // the lane's first column
  uint32_t mk[NMK], mg[NMK];
#pragma unroll
  for (int k = 0; k < NMK; ++k) {
    mk[k] = A.mask[k];
    asm volatile("v_mov_b32 %0, %1" : "=v"(mg[k]) : "s"(A.magic[k]));
  }

  // ---- the weight stream: this wave's K-step of the workgroup's 4-row blocks
  const int RB = (A.N + GV_RPW - 1) / GV_RPW;
  const int b0 = (int)(((long long)RB * blockIdx.x) / gridDim.x);
  const int b1 = (int)(((long long)RB * (blockIdx.x + 1)) / gridDim.x);
  const int nb = b1 - b0;
  const uint32_t wrow = (uint32_t)(A.K / F::WORD_K) * 4u;
  const uint32_t srow = (uint32_t)(A.K / F::G) * 2u;
  const uint32_t woff = (uint32_t)kl / (ONE ? 8u : 4u);   // the lane's code bytes within a row
  const uint32_t soff = (uint32_t)(kl / F::G) * 2u;         // its group's scale within a row
  const char* wq = reinterpret_cast<const char*>(A.w);
  const char* sc = reinterpret_cast<const char*>(A.scales);
  const char* bi = reinterpret_cast<const char*>(A.biases);
  struct GUnit {
    uint32_t w[NWORD];
    uint32_t s, b;
  };
  auto issue = [&](int k, GUnit& R) {
    const int blk = b0 + min(k, nb - 1);
    const int row = min(blk * GV_RPW + rho, A.N - 1);
    const char* p = wq + (size_t)row * wrow + woff;
    if constexpr (ONE) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      R.w[0] = v.x;
      R.w[1] = v.y;
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) R.w[i] = v[i];
    }
    if constexpr (SBI) {   // the group's (scale, bias) word of the interleaved layout
      R.s = *reinterpret_cast<const uint32_t*>(sc + 2 * ((size_t)row * srow + soff));
      R.b = 0;
    } else {
      R.s = *reinterpret_cast<const uint16_t*>(sc + (size_t)row * srow + soff);
      if constexpr (F::AFFINE) R.b = *reinterpret_cast<const uint16_t*>(bi + (size_t)row * srow + soff);
    }
  };
  GUnit ring[PREF];
  // the first units' loads go out right behind the activations', so their latency
  // overlaps the activation set-up below
  auto start_ring = [&]() {
    if (nb > 0) {
#pragma unroll
      for (int d = 0; d < PREF; ++d) issue(d, ring[d]);
    }
  };

  // ---- the lane's activations: 64 columns of each row as raw 16-bit values.  The four lane
  // rows (rho) of a wave need the same columns, so each loads one quarter (32 bytes) and the
  // quarters are exchanged across lane rows afterwards.
  auto load_quarter = [&](int m, u32x4 (&xq)[2]) {
    const uint16_t* p = static_cast<const uint16_t*>(A.x) + (size_t)m * A.K + kl + 16 * rho;
    xq[0] = *reinterpret_cast<const u32x4*>(p);
    xq[1] = *reinterpret_cast<const u32x4*>(p + 8);
  };
  // xr[q] = columns 8q .. 8q+7 of the lane's 64, quarter r = xr[2r], xr[2r+1]: a permlane32
  // swap leaves quarter (rho & 1) in [0] and 2 + (rho & 1) in [1]; a permlane16 swap of each
  // splits those into the even and odd quarters
  auto gather_row = [&](const u32x4 (&xq)[2], u32x4 (&xr)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = xq[h][e];
        const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        const auto lo = __builtin_amdgcn_permlane16_swap(s32[0], s32[0], false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(s32[1], s32[1], false, false);
        xr[0 + h][e] = lo[0];
        xr[2 + h][e] = lo[1];
        xr[4 + h][e] = hi[0];
        xr[6 + h][e] = hi[1];
      }
  };
  u32x4 xq[MM][2];
#pragma unroll
  for (int m = 0; m < MM; ++m) load_quarter(m, xq[m]);
  start_ring();
  float f[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) f[m] = 1.0f;
  if constexpr (NORM) {
    // per-row power of two from the row's largest magnitude over the whole K
    if (tid < MAXM) rowmax[tid] = 0.0f;
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      u16x2 mx2 = {0, 0};   // over the lane's quarter; the wave's lanes cover every column
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, xq[m][q][e] & 0x7FFF7FFFu));
      float mx = half_bits_to_f32<XT>(mx2[0] > mx2[1] ? mx2[0] : mx2[1]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      if (lane == 0) atomicMax(reinterpret_cast<uint32_t*>(rowmax) + m, __float_as_uint(mx));
    }
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float mx = rowmax[m];
      if (mx > 0.0f && mx == mx) {
        int ex = 0;
        frexpf(mx, &ex);
        int e = 14 - ex - (HAD ? 4 : 0);
        e = e < -120 ? -120 : (e > 120 ? 120 : e);
        f[m] = ldexpf(1.0f, e);
      }
    }
  }

  // ---- operand pairs: pair P = wi * HALF + j is (x[WORD_K wi + j], x[WORD_K wi + j + HALF])
  uint32_t xp[MM][32];
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    u32x4 xr[8];
    gather_row(xq[m], xr);
    auto raw = [&](int a) -> uint32_t { return xr[a >> 3][(a >> 1) & 3]; };   // dword holding column a
    if constexpr (HAD) {
      float v[64];
#pragma unroll
      for (int a = 0; a < 64; ++a) {
        const uint32_t d = raw(a);
        v[a] = half_bits_to_f32<XT>((a & 1) ? (d >> 16) : (d & 0xFFFFu));
      }
      if (A.signs) {
        const uint32_t s0 = A.signs[kl >> 5], s1 = A.signs[(kl >> 5) + 1];
#pragma unroll
        for (int a = 0; a < 64; ++a) {
          const uint32_t bit = ((a < 32 ? s0 : s1) >> (a & 31)) & 1u;
          v[a] = __uint_as_float(__float_as_uint(v[a]) ^ (bit << 31));
        }
      }
#pragma unroll
      for (int h = 1; h < 64; h <<= 1)
#pragma unroll
        for (int a = 0; a < 64; ++a)
          if ((a & h) == 0) {
            const float p0 = v[a], p1 = v[a + h];
            v[a] = p0 + p1;
            v[a + h] = p0 - p1;
          }
      // blocks of 128 and 256 span lane pairs (gam ^ 1) and quads (gam ^ 2); each stage
      // leaves the upper lane's results negated, undone by the lane's final sign
      const int cross = A.had_stages - 1;
      if (cross >= 1) {
        const float c1 = (gam & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int a = 0; a < 64; ++a) v[a] = __builtin_fmaf(c1, gv_dpp<0xB1>(v[a]), v[a]);
      }
      if (cross >= 2) {
        const float c2 = (gam & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int a = 0; a < 64; ++a) v[a] = __builtin_fmaf(c2, gv_dpp<0x4E>(v[a]), v[a]);
      }
      const float sg = (__builtin_popcount(gam & ((1 << (cross > 0 ? cross : 0)) - 1)) & 1) ? -1.0f : 1.0f;
      const float sc = sg * A.had_scale * f[m];
#pragma unroll
      for (int wi = 0; wi < NWORD; ++wi)
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int a = F::WORD_K * wi + j;
          xp[m][wi * HALF + j] = f32_to_f16_bits(v[a] * sc) | (f32_to_f16_bits(v[a + HALF] * sc) << 16);
        }
    } else {
#pragma unroll
      for (int wi = 0; wi < NWORD; ++wi)
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int a = F::WORD_K * wi + j, b = a + HALF;
          const uint32_t da = raw(a), db = raw(b);
          if constexpr (NORM) {
            const float fa = __uint_as_float((a & 1) ? (da & 0xFFFF0000u) : (da << 16));
            const float fb = __uint_as_float((b & 1) ? (db & 0xFFFF0000u) : (db << 16));
            xp[m][wi * HALF + j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fa * f[m], fb * f[m]));
          } else {
            xp[m][wi * HALF + j] = __builtin_amdgcn_perm(db, da, (a & 1) ? 0x07060302u : 0x05040100u);
          }
        }
    }
  }
  // ---- the lane's offset and group sums from the same operand values
  float off[MM], xs[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    float e = 0.0f, t = 0.0f;
#pragma unroll
    for (int P = 0; P < NWORD * HALF; ++P) {
      const int j = P % HALF;
      if constexpr (BF) {
        const __bf16 cb = (__bf16)sign1_beta_bf16(j), one = (__bf16)1.0f;
        e = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xp[m][P]), bf16x2{cb, cb}, e, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xp[m][P]), bf16x2{one, one}, t, false);
      } else {
        const float beta = ONE ? sign1_beta(j) : affine2_beta(j);
        const _Float16 cf = (_Float16)beta;
        e = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xp[m][P]), f16x2{cf, cf}, e, false);
        t = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xp[m][P]), f16x2{(_Float16)1.0f, (_Float16)1.0f}, t, false);
      }
    }
    // sign bits decode to BETA + 1 + sign: the offset is sum a (BETA + 1); the affine
    // codes' is sum a BETA
    off[m] = FMT == SIGN1 ? -(e + t) : -e;
    xs[m] = t;
  }

  for (int base = 0; base < nb; base += PREF) {
#pragma unroll
    for (int d = 0; d < PREF; ++d) {
      const int k = base + d;
      if (k < nb) {
        const GUnit R = ring[d];
        if (k + PREF < nb) issue(k + PREF, ring[d]);
        float dot[MM][2];   // two chains per row (even and odd pairs), added at the end
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          dot[m][0] = off[m];
          dot[m][1] = 0.0f;
        }
#pragma unroll
        for (int wi = 0; wi < NWORD; ++wi) {
          uint32_t pw[HALF];
          unpack_word_rt<FMT, BF>(R.w[wi], pw, mk, mg);
#pragma unroll
          for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
              float& d = dot[m][j & 1];
              if constexpr (BF)
                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[j]),
                                                    __builtin_bit_cast(bf16x2, xp[m][wi * HALF + j]), d, false);
              else
                d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw[j]),
                                           __builtin_bit_cast(f16x2, xp[m][wi * HALF + j]), d, false);
            }
        }
        const float s_ = half_of(R.s, 0) * SCALE_MUL;
        const float b_ = F::AFFINE ? (SBI ? half_of(R.s, 1) : half_of(R.b, 0)) : 0.0f;
        float y[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          y[m] = __builtin_fmaf(s_, dot[m][0] + dot[m][1], b_ * xs[m]);
          // the row's 16 lanes: quads (xor 1, xor 2), then mirrored halves of 8 and 16
          y[m] += gv_dpp<0xB1>(y[m]);
          y[m] += gv_dpp<0x4E>(y[m]);
          y[m] += gv_dpp<0x141>(y[m]);
          y[m] += gv_dpp<0x140>(y[m]);
        }
        if (gam == 0) {
#pragma unroll
          for (int m = 0; m < MM; ++m) part[((k * GV_RPW + rho) * S + st) * MM + m] = y[m];
        }
      }
    }
  }
  lds_barrier();
  // ---- each row's K-steps added in step order
  for (int e = tid; e < nb * GV_RPW * MM; e += blockDim.x) {
    const int rl = e / MM, m = e - rl * MM;
    const int row = b0 * GV_RPW + rl;
    if (row < A.N) {
      float sum = 0.0f;
      for (int t = 0; t < S; ++t) sum += part[(rl * S + t) * MM + m];
      A.y[(size_t)m * A.N + row] = sum / f[m];
    }
  }
}

// The kernel names carry the variant name, so a trace shows which variant ran.
template <int FMT, int XT, int PREF, bool EARLY, bool SBI, bool DIRECT, bool SIX, bool DARG>
__global__ __launch_bounds__(NTHREADS) void vg_mfma_q(MfmaArgs A) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  mfma_body<FMT, VAR_MFMA_Q, XT, PREF, false, EARLY, SBI, DIRECT, SIX, DARG>(A, smem);
}
template <int FMT, int XT, int PREF, bool AMASK, bool EARLY, bool SBI, bool DIRECT, bool DARG>
__global__ __launch_bounds__(NTHREADS) void vg_mfma_h(MfmaArgs A) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  mfma_body<FMT, VAR_MFMA_H, XT, PREF, AMASK, EARLY, SBI, DIRECT, false, DARG>(A, smem);
}

// ---------------------------------------------------------------------------------------
// Host side of the MFMA variants.

// The code-extraction masks and magics of unpack_word_rt for a (format, activation dtype)
// pair, built once per call on the host and held in registers by the kernels.  The GEMM
// and the debug decode below take them from here, so the decode the tests check bit for
// bit is the one the GEMM runs.
static void decode_consts(int fmt, int xt, uint32_t mask[8], uint32_t magic[8]) {
  for (int k = 0; k < 8; ++k) {
    if (bf16_codes(fmt, xt)) {
      mask[k] = (1u << k) | (1u << (k + 16));   // positions 0..7
      magic[k] = bf16_magic_sign1(k) | (bf16_magic_sign1(k) << 16);
    } else if (k >= 6) {
      mask[k] = magic[k] = 0u;
    } else if (fmt_one_bit(fmt)) {
      const int q = 5 + k;   // positions 5..10
      mask[k] = (1u << q) | (1u << (q + 16));
      magic[k] = half_magic_sign1(q) | (half_magic_sign1(q) << 16);
    } else {
      const int q = 4 + 2 * (k < 3 ? k : 2);   // positions 4, 6, 8
      mask[k] = (3u << q) | (3u << (q + 16));
      magic[k] = half_magic_affine2(q) | (half_magic_affine2(q) << 16);
    }
  }
}
// Packed-weight bytes of a call (codes, scales and biases).
static double packed_bytes(int fmt, int K, int N) {
  if (fmt == SIGN1) return (double)N * K / 8 + 2.0 * N * K / 128;
  if (fmt == AFFINE1) return (double)N * K / 8 + 4.0 * N * K / 128;
  return (double)N * K / 4 + 4.0 * N * K / 64;
}

// Largest staging window (in K-steps) whose LDS carve-up fits, balanced so the windows of
// a slice of S K-steps have equal step counts; 0 when nothing fits.
static int window_steps(int fmt, int M, int S, int tiles_max, int max_lds, size_t* lds) {
  int best = 0;
  // at most MAXT activation chunks of 32 K per thread: M * ws * KSTEP / 32 <= NTHREADS * MAXT
  const int ws_cap = (NTHREADS * MAXT * 32) / (M * KSTEP);
  for (int ws = S < ws_cap ? S : ws_cap; ws >= 1; --ws) {
    if (LdsLayout(fmt, M, ws, tiles_max).total <= max_lds) { best = ws; break; }
  }
  if (best == 0) return 0;
  const int nwin = (S + best - 1) / best;
  const int ws = (S + nwin - 1) / nwin;
  *lds = (size_t)LdsLayout(fmt, M, ws, tiles_max).total;
  return ws;
}

// The rest of a plan once the row groups and K slices are fixed: tile bound, staging
// window and units in flight.
static bool finish_plan(int fmt, int M, int K, int N, int rg, int ks, const DeviceInfo& dev, MfmaPlan* p) {
  const int S = K / KSTEP;
  p->ks = ks;
  p->rg = rg;
  const int rows_max = (N + rg - 1) / rg + 1;
  if (rows_max > (1 << 18)) return false;   // the output store maps elements to rows by a float reciprocal
  p->tiles_max = (rows_max + 15) / 16 + 1;
  if (p->tiles_max > 32767) return false;   // the split-tile records hold 15-bit tile indices
  if (K >= (1 << 26)) return false;   // lane offsets are 24-bit products of a row and a row's bytes
  // the kernels divide by ks with a multiply-high, exact for n * ks < 2^32 (n <= S * ks)
  if ((uint64_t)(K / KSTEP) * (uint64_t)ks * (uint64_t)ks >= (1ull << 31)) return false;
  const int s_wg = (S + ks - 1) / ks;
  p->win_steps = window_steps(fmt, M, s_wg, p->tiles_max, dev.max_lds, &p->lds);
  // Units in flight per wave: two for the 1-bit formats (their units are half as large),
  // one for the 2-bit formats, long streams included (a second unit in flight measured
  // slower on every 2-bit shape, the 243 MB output head too).
  p->pref = fmt_one_bit(fmt) ? 2 : 1;
  // the fewest units any wave gets: the smallest workgroup's tiles times the K-steps, over NW
  p->direct = ks == 1 && p->win_steps >= S && (N / rg + 15) / 16 * S >= NW * p->pref;
  return p->win_steps > 0;
}

bool plan_mfma(int fmt, int variant, int M, int K, int N, const DeviceInfo& dev, int force_ks, MfmaPlan* p) {
  (void)variant;
  const int tiles = (N + 15) / 16;
  const int S = K / KSTEP;
  const int cus = dev.cu_count;
  // K slices: the count minimising a per-workgroup cost in bytes, which adds the weight
  // units it streams (16-row tiles, so a short last tile costs a whole one), the activation
  // bytes it stages at full weight, double for the rotated format (the transform runs in
  // every workgroup), and for a split the partial outputs
  // written and read back plus a fixed cost for the reduction at the end.  Measured on
  // MI355X against forced slice counts.
  int ks = 1;
  if (force_ks > 0) {
    ks = force_ks < S ? force_ks : S;
  } else {
    const double unit_bytes = packed_bytes(fmt, KSTEP, 16);
    const int ks_max = S < 16 ? S : 16;
    double best = 0.0;
    for (int k = 1; k <= ks_max; ++k) {
      int g = cus / k;
      if (g > tiles) g = tiles;
      if (g < 1) g = 1;
      const int rows = (N + g - 1) / g, steps = (S + k - 1) / k;
      const double stage_weight = fmt == HAD2 ? 2.0 : 1.0;
      double cost = (double)((rows + 15) / 16) * steps * unit_bytes + stage_weight * steps * M * KSTEP * 2.0;
      if (k > 1) cost += 8.0 * k * M * rows + 20480.0;
      if (k == 1 || cost < best) { best = cost; ks = k; }
    }
  }
  int rg = cus / ks;
  if (rg > tiles) rg = tiles;
  if (rg < 1) rg = 1;
  p->grid = rg * ks;
  return finish_plan(fmt, M, K, N, rg, ks, dev, p);
}

bool plan_mfma_grouped(int fmt, int M, int K, int N, int jobs, const DeviceInfo& dev, MfmaPlan* p) {
  // One workgroup per CU (the kernels hold one per CU): at least rg_min row groups for
  // each of the most jobs a routing can make, more when the routing makes fewer.
  const int tiles = (N + 15) / 16;
  int rg_min = (dev.cu_count + jobs - 1) / jobs;
  if (rg_min > tiles) rg_min = tiles;
  p->grid = jobs * rg_min;
  return finish_plan(fmt, M, K, N, rg_min, 1, dev, p);
}

size_t mfma_workspace_bytes(int M, int N, const MfmaPlan& p) {
  return p.ks > 1 ? (size_t)p.ks * M * N * sizeof(float) : 0;
}

// Raises a kernel's dynamic-LDS limit once per device.
static hipError_t allow_lds(void (*kern)(MfmaArgs), std::atomic<uint64_t>& done, const DeviceInfo& dev) {
  const uint64_t bit = 1ull << (dev.id & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, dev.max_lds);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int FMT, int MODE, int XT, int PREF, bool EARLY, bool SBI>
static hipError_t launch_kern(const MfmaArgs& A, const MfmaPlan& p, hipStream_t stream, const DeviceInfo& dev) {
  // 1-bit codes at 8 rows: the A-operand reads of the lanes without a drafted row are
  // masked off (AMASK).  With the zero row those reads carry 4 * 8 + 4 distinct addresses,
  // one more LDS pass per read than the 32 of the drafted rows; the masking costs three
  // scalar instructions per read group, which pays at 8 rows only (measured on MI355X).
  constexpr bool MASKABLE = MODE == VAR_MFMA_H && fmt_one_bit(FMT);
  // The instance whose waves store their tiles without a barrier after the loop (the plan's
  // direct case); every wave of it carries at least PREF units, so its first loads are issued
  // unconditionally.  With the argmax its waves also fold the keys of the tiles they store
  // (DARG).
  const bool direct = p.direct && p.pref == PREF && !A.route;
  const bool darg = direct && A.idx != nullptr;
  // Mode Q issues its first weight loads after the staging, and a wave with no staging chunk
  // sends them out at once.  When one round of a window's chunks would keep seven or eight
  // waves busy, six waves take them (SIX, some in two rounds), so two waves start the weight
  // stream while the others stage: 0.4 to 0.6 us faster at three rows of the 5120-wide
  // shapes on MI355X, where the 480 chunks otherwise occupy all eight waves.  Level or slower
  // at every other count measured.
  const int chunks = A.M * (p.win_steps * KSTEP / 32);
  const bool six = MODE == VAR_MFMA_Q && !A.route && chunks > 6 * 64 && chunks <= NTHREADS;
  bool amask = false;
  void (*kern)(MfmaArgs);
  if constexpr (MODE == VAR_MFMA_Q) {
    if (!direct)
      kern = six ? vg_mfma_q<FMT, XT, PREF, EARLY, SBI, false, true, false> : vg_mfma_q<FMT, XT, PREF, EARLY, SBI, false, false, false>;
    else if (darg)
      kern = six ? vg_mfma_q<FMT, XT, PREF, EARLY, SBI, true, true, true> : vg_mfma_q<FMT, XT, PREF, EARLY, SBI, true, false, true>;
    else
      kern = six ? vg_mfma_q<FMT, XT, PREF, EARLY, SBI, true, true, false> : vg_mfma_q<FMT, XT, PREF, EARLY, SBI, true, false, false>;
  } else {
    kern = !direct ? vg_mfma_h<FMT, XT, PREF, false, EARLY, SBI, false, false>
                   : (darg ? vg_mfma_h<FMT, XT, PREF, false, EARLY, SBI, true, true>
                           : vg_mfma_h<FMT, XT, PREF, false, EARLY, SBI, true, false>);
    if constexpr (MASKABLE) {
      if (A.M == 8) {
        amask = true;
        kern = !direct ? vg_mfma_h<FMT, XT, PREF, true, EARLY, SBI, false, false>
                       : (darg ? vg_mfma_h<FMT, XT, PREF, true, EARLY, SBI, true, true>
                               : vg_mfma_h<FMT, XT, PREF, true, EARLY, SBI, true, false>);
      }
    }
  }
  static std::atomic<uint64_t> attr_done[2][2][2][2];
  std::atomic<uint64_t>* done = &attr_done[amask][direct][six][darg];
  const hipError_t e = allow_lds(kern, *done, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(NTHREADS), p.lds, stream, A);
  return hipGetLastError();
}

template <int FMT, int MODE, int XT, bool SBI>
static hipError_t launch_one(const GemmCall& c, const MfmaPlan& p, float* part, uint32_t* counters,
                             const DeviceInfo& dev) {
  if (p.win_steps <= 0 || (p.ks > 1 && (part == nullptr || counters == nullptr))) return hipErrorInvalidValue;
  MfmaArgs A{};
  A.x = c.x; A.w = c.w; A.scales = c.scales; A.biases = c.biases; A.y = c.y;
  A.M = c.M; A.K = c.K; A.N = c.N;
  A.win_steps = p.win_steps;
  A.tiles_max = p.tiles_max;
  A.a_pitch = p.win_steps * fmt_gps(FMT) * fmt_gs(FMT) + 16;
  A.rg = p.rg;
  A.ks = p.ks;
  A.rq = c.N / p.rg;
  A.rrem = c.N - A.rq * p.rg;
  A.ks_magic = p.ks > 1 ? (uint32_t)(((1ull << 32) + (uint64_t)p.ks - 1) / (uint64_t)p.ks) : 0u;
  A.ws_magic = p.win_steps > 1 ? (uint32_t)(((1ull << 32) + (uint64_t)p.win_steps - 1) / (uint64_t)p.win_steps) : 0u;
  A.lay = LdsLayout(FMT, c.M, p.win_steps, p.tiles_max);
  A.part = part;
  A.counters = counters;
  A.route = c.route;
  A.topk = c.topk;
  A.E = c.E;
  A.cap = c.cap;
  A.w_estride = c.w_estride;
  A.s_estride = c.s_estride;
  A.idx = c.idx;
  A.draft = c.draft;
  A.accepted = c.accepted;
  A.amax_key = c.amax_key;
  A.had_stages = c.had_block == 64 ? 1 : (c.had_block == 256 ? 3 : 2);
  A.had_scale = c.had_block == 64 ? 0.125f : (c.had_block == 256 ? 0.0625f : 0.08838834764831845f);
  A.signs = c.signs;
  decode_consts(FMT, XT, A.mask, A.magic);
  // Mode H (5 to 8 rows) issues a wave's first weight loads as soon as its own activation
  // loads have landed, so the weight latency overlaps the staging arithmetic; mode Q, and
  // the rotated format's longer staging, issue them after it (each order measured faster
  // there on MI355X).
  constexpr bool EARLY = MODE == VAR_MFMA_H && FMT != HAD2;
  if constexpr (fmt_one_bit(FMT)) return launch_kern<FMT, MODE, XT, 2, EARLY, SBI>(A, p, c.stream, dev);
  else return launch_kern<FMT, MODE, XT, 1, EARLY, SBI>(A, p, c.stream, dev);
}

hipError_t launch_mfma(const GemmCall& c, int variant, const MfmaPlan& p, float* part, uint32_t* counters,
                       const DeviceInfo& dev) {
#define VG_DISPATCH_SBI(FMT, MODE, XT)                                                         \
  if constexpr (FMT != SIGN1) {                                                                \
    if (c.sbi) return launch_one<FMT, MODE, XT, true>(c, p, part, counters, dev);              \
  }                                                                                            \
  return launch_one<FMT, MODE, XT, false>(c, p, part, counters, dev);
#define VG_DISPATCH_XT(FMT, MODE)                                                   \
  switch (c.xt) {                                                                    \
    case XF16: { VG_DISPATCH_SBI(FMT, MODE, XF16) }                                  \
    case XBF16: { VG_DISPATCH_SBI(FMT, MODE, XBF16) }                                \
    default: return hipErrorInvalidValue;                                            \
  }
#define VG_DISPATCH_MODE(FMT)                                                       \
  if (variant == VAR_MFMA_Q) { VG_DISPATCH_XT(FMT, VAR_MFMA_Q) }                     \
  else { VG_DISPATCH_XT(FMT, VAR_MFMA_H) }
  switch (c.fmt) {
    case SIGN1: VG_DISPATCH_MODE(SIGN1)
    case AFFINE2: VG_DISPATCH_MODE(AFFINE2)
    case HAD2: VG_DISPATCH_MODE(HAD2)
    case AFFINE1: VG_DISPATCH_MODE(AFFINE1)
    default: return hipErrorInvalidValue;
  }
#undef VG_DISPATCH_MODE
#undef VG_DISPATCH_XT
#undef VG_DISPATCH_SBI
}

// The dot2 kernel: one wave per 1024-wide K-step (K <= 16384), rows one or two (one for the
// rotated format, whose transform needs the registers); enough
// workgroups for about 20 waves per CU, each a balanced range of 4-row blocks whose
// per-step partials fit the LDS.
bool plan_gemv(int fmt, int M, int K, int N, const DeviceInfo& dev, MfmaPlan* p) {
  if (M < 1 || M > (fmt == HAD2 ? 1 : 2) || K % KSTEP != 0 || N < 1) return false;
  const int S = K / KSTEP;
  if (S > GV_MAXS) return false;
  const int rb = (N + GV_RPW - 1) / GV_RPW;
  int grid = (dev.cu_count * 20 + S - 1) / S;
  if (grid > rb) grid = rb;
  const int nb_max = (rb + grid - 1) / grid;
  const size_t lds = (size_t)2 * MAXM * 4 + (size_t)nb_max * GV_RPW * S * M * 4;
  if (lds > (size_t)dev.max_lds) return false;
  p->grid = grid;
  p->rg = grid;
  p->ks = 1;
  p->win_steps = S;
  p->tiles_max = 0;
  p->pref = 3;
  p->lds = lds;
  p->direct = false;
  return true;
}

// The grid is one round of resident workgroups: the plan's wave count per CU, cut to what
// the instance's registers allow (a second round would start after the first has drained).
template <int FMT, int XT, int MM, bool SBI>
static hipError_t launch_gemv_m(const MfmaArgs& A, const MfmaPlan& p, hipStream_t stream, const DeviceInfo& dev) {
  void (*kern)(MfmaArgs) = vg_gemv<FMT, XT, MM, 3, SBI>;
  static std::atomic<uint64_t> attr_done{0};
  static std::atomic<int> resident[8][GV_MAXS + 1];   // workgroups per CU by device and S (0: unknown)
  hipError_t e = allow_lds(kern, attr_done, dev);
  if (e != hipSuccess) return e;
  const int S = p.win_steps;
  std::atomic<int>& slot = resident[dev.id & 7][S];
  int per_cu = slot.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * S, p.lds);
    if (e != hipSuccess) return e;
    // a workgroup's waves do not always spread evenly over the 4 SIMDs: two waves of
    // headroom per CU keep the whole grid resident at once.  At most 16 waves per CU: at
    // K = 5120 (5 waves a workgroup) 3 workgroups per CU ran 0.4-0.6 us ahead of 2 and of
    // 4 (measured on MI355X), and the interleaved-metadata instances, with fewer
    // registers, would otherwise get 4.
    const int regs = fa.numRegs < 8 ? 8 : ((fa.numRegs + 7) / 8) * 8;
    const int wps = std::min(8, 512 / regs);
    const int waves_max = std::min(4 * wps - 2, 16);
    while (per_cu > 1 && per_cu * S > waves_max) --per_cu;
    per_cu = per_cu < 1 ? 1 : per_cu;
    slot.store(per_cu, std::memory_order_relaxed);
  }
  int grid = p.grid;
  size_t lds = p.lds;
  if (grid > per_cu * dev.cu_count) {
    grid = per_cu * dev.cu_count;
    const int rb = (A.N + GV_RPW - 1) / GV_RPW;
    lds = (size_t)2 * MAXM * 4 + (size_t)((rb + grid - 1) / grid) * GV_RPW * S * MM * 4;
    if (lds > (size_t)dev.max_lds) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * S), lds, stream, A);
  return hipGetLastError();
}

template <int FMT, int XT, bool SBI>
static hipError_t launch_gemv_x(const GemmCall& c, const MfmaPlan& p, const DeviceInfo& dev) {
  MfmaArgs A{};
  A.x = c.x; A.w = c.w; A.scales = c.scales; A.biases = c.biases; A.y = c.y;
  A.M = c.M; A.K = c.K; A.N = c.N;
  A.had_stages = c.had_block == 64 ? 1 : (c.had_block == 256 ? 3 : 2);
  A.had_scale = c.had_block == 64 ? 0.125f : (c.had_block == 256 ? 0.0625f : 0.08838834764831845f);
  A.signs = c.signs;
  decode_consts(FMT, XT, A.mask, A.magic);
  if (c.M == 1) return launch_gemv_m<FMT, XT, 1, SBI>(A, p, c.stream, dev);
  if constexpr (FMT != HAD2) {   // two rotated rows do not fit the kernel's registers
    if (c.M == 2) return launch_gemv_m<FMT, XT, 2, SBI>(A, p, c.stream, dev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemmCall& c, const MfmaPlan& p, const DeviceInfo& dev) {
#define VG_GEMV_SBI(FMT, XT)                                             \
  if constexpr (FMT != SIGN1) {                                          \
    if (c.sbi) return launch_gemv_x<FMT, XT, true>(c, p, dev);           \
  }                                                                      \
  return launch_gemv_x<FMT, XT, false>(c, p, dev);
#define VG_GEMV_XT(FMT)                                                  \
  switch (c.xt) {                                                        \
    case XF16: { VG_GEMV_SBI(FMT, XF16) }                                \
    case XBF16: { VG_GEMV_SBI(FMT, XBF16) }                              \
    default: return hipErrorInvalidValue;                                \
  }
  switch (c.fmt) {
    case SIGN1: VG_GEMV_XT(SIGN1)
    case AFFINE2: VG_GEMV_XT(AFFINE2)
    case HAD2: VG_GEMV_XT(HAD2)
    case AFFINE1: VG_GEMV_XT(AFFINE1)
    default: return hipErrorInvalidValue;
  }
#undef VG_GEMV_XT
#undef VG_GEMV_SBI
}

hipError_t launch_debug_decode(int fmt, int xt, const uint32_t* w, int N, int K, uint8_t* codes, hipStream_t s) {
  DecodeArgs D;
  D.w = w;
  D.codes = codes;
  D.N = N;
  D.K = K;
  decode_consts(fmt, xt, D.mask, D.magic);
  const size_t words = (size_t)N * (size_t)(K / fmt_word_k(fmt));
  if (words == 0 || (words + 255) / 256 > 0x7FFFFFFFu) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((words + 255) / 256));
  const bool bf = bf16_codes(fmt, xt);
  switch (fmt) {
    case SIGN1:
      if (bf) hipLaunchKernelGGL((vg_debug_decode<SIGN1, true>), grid, dim3(256), 0, s, D);
      else hipLaunchKernelGGL((vg_debug_decode<SIGN1, false>), grid, dim3(256), 0, s, D);
      break;
    case AFFINE1:
      if (bf) hipLaunchKernelGGL((vg_debug_decode<AFFINE1, true>), grid, dim3(256), 0, s, D);
      else hipLaunchKernelGGL((vg_debug_decode<AFFINE1, false>), grid, dim3(256), 0, s, D);
      break;
    case AFFINE2: hipLaunchKernelGGL((vg_debug_decode<AFFINE2, false>), grid, dim3(256), 0, s, D); break;
    case HAD2: hipLaunchKernelGGL((vg_debug_decode<HAD2, false>), grid, dim3(256), 0, s, D); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Static scratch of the allocation-free entry point (verify_gemm_argmax_noalloc): the
// split-K partials, arrival counters and argmax keys of a call in a fixed device array,
// one copy per GPU the library runs on, held until the process ends.  In host code the
// array's name is a host-side stand-in, not a device address: its address on a device is
// taken once per device with hipGetSymbolAddress (that device current), and only that
// address reaches kernels.  Calls on one GPU share the array, so calls that overlap on one
// GPU race; the kernels leave the counters zero for the next call.
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void vg_clear_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

hipError_t static_scratch(int dev, size_t clear_bytes, hipStream_t s, char** out) {
  static std::mutex mu;
  static char* ptr[64] = {};
  if (dev < 0 || dev >= 64 || clear_bytes > STATIC_SCRATCH_BYTES || clear_bytes % 4) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // The counters must read zero before the first call.  The array is zero when the code
    // object loads and every call leaves its counters zero; they are cleared once here
    // regardless, by a kernel (no memset node, should the first call be captured).
    hipLaunchKernelGGL(vg_clear_words, dim3(64), dim3(256), 0, s, static_cast<uint32_t*>(p),
                       (uint32_t)(clear_bytes / 4));
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    ptr[dev] = static_cast<char*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace vg
