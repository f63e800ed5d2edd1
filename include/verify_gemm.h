/*
 * verify_gemm.h -- C ABI of the few-row quantized verify GEMM for MI355X (gfx950).
 *
 * Speculative decoding checks a block of M drafted rows in one target pass.  The verify
 * GEMM multiplies those M <= 8 activation rows against packed low-bit weights, decoding
 * each weight once inside the contraction and never writing a dense copy, so the cost is
 * nearly flat in M ("Ishizuki" README, section "Kernels written for the verify";
 * "dflash-mlx-bonsai2" README, sections "Why" and "What this fork adds").
 *
 * Conventions shared by every entry point
 *   - Pointers named x, w*, scales, biases, y, x_out, idx, codes are DEVICE pointers owned
 *     by the caller.  The library never frees or keeps them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work and return; results are valid once the caller synchronizes the stream.
 *   - Arguments are validated on the host before anything is enqueued.  On error the call
 *     returns a non-zero vg_status, enqueues nothing, and vg_last_error() returns a message
 *     (per calling thread).
 *   - The library keeps a small read-only per-device state (device attributes) created on
 *     first use.  The GEMM calls allocate no device memory, except that a call whose K
 *     the dispatch splits across workgroups (see vg_plan_ksplit), and the argmax and
 *     acceptance calls, use a workspace owned by the library: one per device and stream,
 *     created on the first such call on that stream (hipMalloc, and a clear of its
 *     counters enqueued on the stream) and replaced by a larger one when a call needs
 *     more.  A replaced workspace is not freed while the process runs (enqueued work or a
 *     captured graph may still use it); vg_release_stream_workspace frees a stream's
 *     workspaces.  The kernels leave the workspace's counters zero, so calls on
 *     one stream share it in stream order; calls on different streams use different
 *     workspaces.  There is no limit on the number of streams.
 *   - HIP graph capture: a call whose workspace already exists at the size it needs (one
 *     earlier eager call of the same kind and no smaller size on the stream) enqueues
 *     kernel launches only and can be captured and replayed.  A call under capture that
 *     would need to create or grow its workspace is refused with VG_ERR_UNSUPPORTED
 *     before anything is enqueued.  A replay uses the workspace of the stream the call was
 *     captured on: replays must be ordered with each other and with eager calls on that
 *     stream (replay on that stream, or synchronize), since overlapping calls would share
 *     its counters.
 *   - Host threads: calls may come from any thread; calls that share a stream are ordered
 *     by that stream.
 *   - Activations x are row-major [M, K] of dtype VG_F32, VG_F16 or VG_BF16 (raw IEEE bits);
 *     outputs y are row-major fp32 [M, N]; rows >= M are never read or written.
 *     VG_BF16 activations against the 1-bit formats enter the matrix cores unscaled,
 *     and their fp32 sums carry per-group offsets of up to 2^15 times an activation: such
 *     activations must stay below 2^110 in magnitude (larger ones give non-finite
 *     outputs).  Every other combination is bounded by fp32's range alone.
 *   - Packed weights, row-major over the N output rows, little-endian words, LSB first:
 *       1-bit sign:  wbits[N, K/32] uint32; weight k of a row is bit k%32 of word k/32;
 *                    bit 0 -> -scale, bit 1 -> +scale; one fp16 scale per 128 weights,
 *                    scales[N, K/128] ("Bonsai-27B-mlx-1bit" model card, binary weight
 *                    format).
 *       2-bit affine: wq[N, K/16] uint32; code k is bits 2(k%16)..2(k%16)+1 of word k/16;
 *                    w = q*s + b with one fp16 scale and one fp16 bias per 64 weights,
 *                    scales[N, K/64], biases[N, K/64] (MLX grouped affine format: a scale
 *                    and a bias per group; same model card, MLX paragraph).
 *   - The affine formats (2-bit, rotated 2-bit, 1-bit affine) also take their scales and
 *     biases interleaved: pass biases = NULL and scales as uint16 [N, K/G, 2], each group's
 *     (scale, bias) pair side by side, scale first (one 32-bit word per group, the scale in
 *     its low half), built once from the two arrays by vg_pack_scale_bias.  The values and
 *     every result are the same bit for bit; the kernels then fetch a lane's scales and
 *     biases with one load instead of one per array, which is faster (the library's
 *     preferred layout).  Grouped expert calls take [E, N, K/G, 2].
 *   - x, weights, scales, biases and y must be 16-byte aligned (whole-word vector loads).
 */
#ifndef VERIFY_GEMM_H
#define VERIFY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VG_OK = 0,
  VG_ERR_ARG = 1,          /* null pointer, unknown enum, bad count                         */
  VG_ERR_SHAPE = 2,        /* M outside 1..8, N < 1, K not a multiple of the group          */
  VG_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned                              */
  VG_ERR_DTYPE = 4,        /* activation dtype not one of vg_dtype                          */
  VG_ERR_UNSUPPORTED = 5,  /* a transform the library cannot apply (e.g. Hadamard block
                              other than 128): refused, never run as the plain format       */
  VG_ERR_HIP = 6           /* the HIP runtime reported an error while enqueueing            */
} vg_status;

typedef enum { VG_F32 = 0, VG_F16 = 1, VG_BF16 = 2 } vg_dtype;

typedef enum { VG_FMT_SIGN1 = 0, VG_FMT_AFFINE2 = 1, VG_FMT_HAD2 = 2, VG_FMT_AFFINE1 = 3 } vg_format;

/* Maximum drafted rows per call (verify blocks of up to 8 rows are padded to 8:
   "dflash-mlx-bonsai2" README, "What this fork adds"). */
#define VG_MAX_ROWS 8

/*
 * y[M, N] = x[M, K] * W^T with W the 1-bit sign g128 weights.
 * Requires 1 <= M <= 8, N >= 1, K >= 128, K % 128 == 0.
 * Source: "Bonsai-27B-mlx-1bit" model card (each weight one sign bit, 0 -> -scale,
 * 1 -> +scale, one FP16 scale per group of 128 weights).
 */
vg_status verify_gemm_sign1(const void* x, int x_dtype, int M, int K,
                            const uint32_t* wbits, const uint16_t* scales, int N,
                            float* y, void* stream);

/*
 * y[M, N] = x[M, K] * W^T with W MLX's 1-bit affine weights: w = c*s + b with a 1-bit code
 * c (0/1) and one fp16 scale s and fp16 bias b per 128 weights (1.25 bits per weight).
 * wbits[N, K/32] packed like the sign bits; scales and biases [N, K/128] fp16.  The sign
 * format is the special case s = 2*s_sign, b = -s_sign.
 * Requires 1 <= M <= 8, N >= 1, K >= 128, K % 128 == 0.
 * Source: "Bonsai-27B-mlx-1bit" model card, MLX paragraph (MLX stores the binary weights
 * as 1-bit affine codes with scale 2s and bias -s per group of 128).
 */
vg_status verify_gemm_affine1(const void* x, int x_dtype, int M, int K,
                              const uint32_t* wbits, const uint16_t* scales,
                              const uint16_t* biases, int N, float* y, void* stream);

/*
 * y[M, N] = x[M, K] * W^T with W the 2-bit affine g64 weights, w = q*s + b.
 * Requires 1 <= M <= 8, N >= 1, K >= 64, K % 64 == 0.
 * Source: MLX grouped affine codes ("Ishizuki" README, "Kernels written for the verify":
 * the verify kernel for MLX affine codes; scale and bias per group: "Bonsai-27B-mlx-1bit"
 * model card, MLX paragraph).
 */
vg_status verify_gemm_affine2(const void* x, int x_dtype, int M, int K,
                              const uint32_t* wq, const uint16_t* scales,
                              const uint16_t* biases, int N, float* y, void* stream);

/*
 * y[M, N] = (x[M, K] * H_bd) * W^T with H_bd block-diagonal, each block the normalized
 * Sylvester Hadamard H_B / sqrt(B), B = had_block, and W 2-bit affine g64 as above.  The
 * rotation runs inside the GEMM's prologue on each workgroup's activations; no rotated
 * copy of x is written.  had_block must be 64, 128 or 256 (anything else ->
 * VG_ERR_UNSUPPORTED: a transform that cannot be applied is refused, never run as the plain
 * format).  Requires 1 <= M <= 8, N >= 1, K % 128 == 0 and K % had_block == 0.
 * Source: "dflash-mlx-bonsai2" README, "What this fork adds" (Hadamard-rotated 2-bit pack,
 * verify GEMM with the Hadamard fused into its prep; the block of the test packs is 128);
 * "Ishizuki" README (a pack declaring a transform that cannot be applied is refused).
 */
vg_status verify_gemm_had2(const void* x, int x_dtype, int M, int K,
                           const uint32_t* wq, const uint16_t* scales,
                           const uint16_t* biases, int N, int had_block, float* y,
                           void* stream);

/*
 * As verify_gemm_had2 with a random sign flip before the rotation:
 * y = ((x * D) * H_bd) * W^T, D = diag(d_k), d_k = -1 where bit k%32 of signs[k/32] is set,
 * +1 elsewhere.  signs is a device array of K/32 uint32 (4-byte aligned), or NULL for
 * verify_gemm_had2.  Source: "dflash-mlx-bonsai2" README, "What this fork adds" (the fused
 * prep names a sign step next to the Hadamard; the pages do not define it, and this
 * diagonal-before-rotation form is the usual randomized Hadamard).
 */
vg_status verify_gemm_had2_signed(const void* x, int x_dtype, int M, int K,
                                  const uint32_t* wq, const uint16_t* scales,
                                  const uint16_t* biases, int N, int had_block,
                                  const uint32_t* signs, float* y, void* stream);

/*
 * x_out[M, K] (fp32) = x[M, K] * H_bd, the same block-B normalized Sylvester rotation as
 * verify_gemm_had2 (B = block: 64, 128 or 256), as a standalone call: the rotation step of
 * the activation prep that the "dflash-mlx-bonsai2" README ("What this fork adds") fuses
 * ahead of the rotated-weight product, here on its own for callers that rotate once and
 * verify several times.  Requires 1 <= M <= 8, K % block == 0.
 */
vg_status hadamard_rotate(const void* x, int x_dtype, int M, int K, int block,
                          float* x_out, void* stream);

/* hadamard_rotate with the sign flip of verify_gemm_had2_signed first (signs may be NULL). */
vg_status hadamard_rotate_signed(const void* x, int x_dtype, int M, int K, int block,
                                 const uint32_t* signs, float* x_out, void* stream);

/*
 * idx[m] = argmax_n y[m, n] for m < M (lowest n on ties; NaN never wins; a row of only
 * NaN gives 0), for the output head of a verify pass ("dflash-mlx-bonsai2" README, "Verify
 * it yourself": the verify is checked by its argmax).  y is fp32 [M, N] row-major (4-byte
 * aligned), idx is int32 [M].  Requires 1 <= M <= 8, N >= 1.  Uses the per-stream workspace
 * described above (the argmax of each row is split over the whole chip).
 */
vg_status verify_argmax_rows(const float* y, int M, int N, int32_t* idx, void* stream);

/*
 * The verify GEMM of one format followed by the argmax of every output row, as one call:
 * y as verify_gemm_<format> computes it, idx[m] = argmax_n y[m, n] as verify_argmax_rows
 * computes it, and with draft non-null accepted[0] as verify_accept_greedy computes it (the
 * output head's verify is checked by its argmax: "dflash-mlx-bonsai2" README, "Verify it
 * yourself").  When the dispatch runs the MFMA kernels with K in one slice (the output-head
 * shapes), the argmax is fused into the GEMM's epilogue: each workgroup stores its
 * columns' best (value, column) per row as one 64-bit key, and one small kernel after the
 * GEMM takes the maximum key of every row over the workgroups and writes idx (and
 * accepted), so the logits are not read back.  Otherwise the argmax kernel runs after the
 * GEMM on the same stream.  Results are identical either way (the argmax rule is
 * order-independent).
 *   format  VG_FMT_SIGN1, VG_FMT_AFFINE2, VG_FMT_HAD2 (block 128, unsigned) or
 *           VG_FMT_AFFINE1; w, scales, biases as in that format's call (biases unused and
 *           may be NULL for VG_FMT_SIGN1; NULL for the interleaved layout otherwise).
 *   y       fp32 [M, N], written as by the plain call.
 *   idx     int32 [M] on the device (4-byte aligned).
 *   draft, accepted  both NULL, or int32 [M] and int32 [1] on the device.
 * Requirements and errors as the format's call, plus idx non-null.  Uses the per-stream
 * workspace described above (allocated on the first call on a stream that needs it).
 */
vg_status verify_gemm_argmax(int format, const void* x, int x_dtype, int M, int K, const uint32_t* w,
                             const uint16_t* scales, const uint16_t* biases, int N, float* y, int32_t* idx,
                             const int32_t* draft, int32_t* accepted, void* stream);

/*
 * verify_gemm_argmax for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, same
 * kernels and plan, so y, idx and accepted are bit for bit those of verify_gemm_argmax;
 * with idx NULL (and draft, accepted NULL) only y is computed, bit for bit the plain
 * verify_gemm_<format> call.  Differences:
 *   - The call's scratch (split-K partial outputs, arrival counters, argmax keys) lives in
 *     a static device array of 4 MiB per GPU, held until the process ends, instead of a
 *     per-stream workspace.  A call that needs more -- 116736 bytes of counters plus the
 *     larger of (K slices) * M * N * 4 bytes of partials (vg_plan_ksplit; none when 1) and,
 *     when the argmax runs as its own kernel after the GEMM, 128 * M * ceil(N / 2048)
 *     bytes of keys, or for the fused argmax 64 bytes of keys per GEMM workgroup (one
 *     workgroup per compute unit at most) -- is refused with VG_ERR_UNSUPPORTED before
 *     anything is enqueued.
 *   - Nothing is allocated and no memset is enqueued.  The first call on a device that
 *     uses the array looks up its address and enqueues one small kernel that clears its
 *     counters; every call leaves them zero for the next.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 *     other streams, or graph replays running beside them) race and give wrong results,
 *     so order them.
 */
vg_status verify_gemm_argmax_noalloc(int format, const void* x, int x_dtype, int M, int K, const uint32_t* w,
                                     const uint16_t* scales, const uint16_t* biases, int N, float* y,
                                     int32_t* idx, const int32_t* draft, int32_t* accepted, void* stream);

/*
 * Greedy acceptance of a drafted block ("dflash-mlx-bonsai2" README, "Verify it yourself":
 * the target's greedy argmax decides which drafted tokens stand): idx[m] = argmax_n y[m, n]
 * as verify_argmax_rows, and accepted[0] = the number of leading rows m with
 * idx[m] == draft[m] (0..M), i.e. the length of the drafted prefix the target model agrees
 * with; when it is below M, idx[accepted[0]] is the target's own token at the first
 * disagreement.  draft is int32
 * [M] on the device; accepted is int32 [1] on the device.  Same requirements as
 * verify_argmax_rows; draft and accepted must be non-null.
 */
vg_status verify_accept_greedy(const float* y, int M, int N, const int32_t* draft, int32_t* idx,
                               int32_t* accepted, void* stream);

/*
 * Grouped routed-expert verify: for a mixture-of-experts layer whose M drafted rows are
 * each routed to topk of E experts, y[m, s, :] = x[m, :] * W_e^T with e = route[m, s], for
 * every routed slot, in one call that reads each routed expert's packed weights once
 * however many rows it serves, and whose output for a slot is bit-identical whichever
 * other rows are routed with it ("Ijah" README, "What's new (v0.2)": grouped routed-expert
 * verify kernels).
 *   format  VG_FMT_SIGN1, VG_FMT_AFFINE2, VG_FMT_HAD2 (block 128, unsigned) or
 *           VG_FMT_AFFINE1; the weights of each expert as in that format's call.
 *   x       activations [M, K], VG_F16 or VG_BF16 (VG_F32 is refused: VG_ERR_UNSUPPORTED).
 *   route   int32 [M, topk] on the device: the expert of each (row, slot); a value outside
 *           0..E-1 marks an unused slot.  Read by the device, so it is not validated on
 *           the host; the call never reads or writes out of bounds whatever it holds.
 *   w, scales, biases  the E experts' packed weights stacked expert-major: w[E, N, words
 *           per row], scales and biases [E, N, groups per row] (biases unused and may be
 *           NULL for VG_FMT_SIGN1; NULL with interleaved scales [E, N, groups per row, 2]
 *           for the affine formats).
 *   y       fp32 [M, topk, N]; the rows of unused slots are not written.
 * Requires 1 <= M <= 8, 1 <= topk <= 8, E >= 1, N >= 1, K a multiple of 1024.  One kernel
 * launch; no workspace.
 */
vg_status verify_gemm_experts(int format, const void* x, int x_dtype, int M, int K, int E, int topk,
                              const int32_t* route, const uint32_t* w, const uint16_t* scales,
                              const uint16_t* biases, int N, float* y, void* stream);

/*
 * Builds the interleaved scale-and-bias layout described above, once, when the weights are
 * loaded: out[2i] = scales[i], out[2i + 1] = biases[i] for 0 <= i < count (count = the
 * number of groups, N * K / G, or E * N * K / G for stacked experts).  The pairs are the
 * MLX grouped affine format's own scale and bias per group ("Bonsai-27B-mlx-1bit" model
 * card, MLX paragraph) in another order; nothing is computed.  scales and biases are
 * uint16 [count], out is uint16 [2 * count], all on the device and 16-byte aligned; out
 * must not overlap either input.  count 0 enqueues nothing.  VG_ERR_SHAPE for count < 0,
 * VG_ERR_ARG for a null or overlapping buffer.
 */
vg_status vg_pack_scale_bias(const uint16_t* scales, const uint16_t* biases, long long count, uint16_t* out,
                             void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* vg_last_error(void);

/*
 * Frees the current device's workspace(s) of `stream` (the split-K partials, arrival
 * counters and argmax keys described above), after synchronizing the stream; VG_OK when
 * the stream has none.  A later call on the stream creates a new one.  Must not be
 * called while work that uses them may still run elsewhere (a graph captured on the
 * stream and replayed later would use freed memory), and is refused (VG_ERR_UNSUPPORTED)
 * while the stream is capturing.  For callers that create and destroy many streams.
 */
vg_status vg_release_stream_workspace(void* stream);

/*
 * Kernel variant the per-shape dispatch picks for a plain verify call of (format, x_dtype,
 * M, N, K), or -1 if the shape is invalid.  A call that also computes the rows' argmax
 * (verify_gemm_argmax) keeps one row on the MFMA kernel whose epilogue fuses the argmax
 * instead of vg_gemv.  vg_variant_name() gives the variant's name, which is also the
 * kernel's name prefix in a rocprofv3 trace.
 */
int vg_plan_variant(int format, int x_dtype, int M, int N, int K);
const char* vg_variant_name(int variant);

/*
 * Force a variant for later calls on this process (tests and A/B timing); -1 restores
 * the dispatch.  Returns VG_ERR_ARG for an unknown variant.  A forced variant that does
 * not support a call's (format, dtype, M) makes that call fail with VG_ERR_UNSUPPORTED.
 */
vg_status vg_force_variant(int variant);

/* Number of variants; variant ids are 0 .. vg_variant_count()-1. */
int vg_variant_count(void);

/*
 * K slices the MFMA variants split a call into (1: each workgroup runs the whole K range
 * of its output rows), or -1 for an invalid shape.  A workgroup stages the activations of
 * its K range once per call; when that staging would exceed the packed bytes it streams,
 * K is split across workgroups, each stages its slice, and the last slice of a row group
 * to finish adds the partial outputs in slice order, so results do not depend on timing.
 */
int vg_plan_ksplit(int format, int x_dtype, int M, int N, int K);

/*
 * Force the K slices of later MFMA calls in this process (tests and timing); 0 restores
 * the dispatch.  Values above K/1024 are capped.  VG_ERR_ARG outside 0..64.
 */
vg_status vg_force_ksplit(int ksplit);

/*
 * How a verify call on vg_plan_variant's MFMA variants (plain, or with the fused argmax of
 * verify_gemm_argmax) finishes its output tiles: 1 when each 16-row tile goes to y from the
 * wave that completes it, with no workgroup barrier after the main loop -- a tile that waves
 * share is added up, in wave order, by the last of them to arrive, and with the argmax each
 * wave folds the keys of the tiles it stores and the workgroup's last wave stores them --
 * and 0 when the waves meet at a barrier and the shared tiles are added up after it (the
 * dot2 and VALU kernels, calls that split K or stage K in more than one window, and
 * workgroups whose waves could get fewer units than they load ahead).  The sum is the same in both, so the outputs are bit-identical.  -1 for
 * arguments no call accepts.  The dispatch is the one the calls make (forced variant and K
 * slices included).
 */
int vg_plan_direct(int format, int x_dtype, int M, int N, int K);

/*
 * Force later MFMA calls in this process (plain and argmax calls) to finish every tile after
 * the workgroup barrier (1), or restore the dispatch (0): tests compare the two finishes bit
 * for bit.  VG_ERR_ARG for other values.
 */
vg_status vg_force_barrier_tail(int on);

/*
 * Measurement aid: a plain streaming read of `bytes` (a positive multiple of 16) from the
 * 16-byte aligned device buffer `buf`, every byte read once with 16-byte non-temporal
 * loads.  Not part of the method: timed at the byte count of a verify call, it shows the
 * bandwidth a kernel doing nothing but reading those bytes reaches on this device, the
 * ceiling beside which the verify GEMM's fraction of the HBM peak is read.
 * vg_stream_read_config takes the loads in flight per thread (1, 2, 4, 8 or 16) and the
 * workgroups of 256 threads per CU (1..32), so the ceiling can be swept; vg_stream_read is
 * the configuration (4, 8).  Each writes one word per workgroup to sink (uint32, device,
 * 4-byte aligned, vg_stream_read_blocks() words).  Validation as elsewhere: VG_ERR_ARG,
 * VG_ERR_ALIGN, VG_ERR_SHAPE.
 */
int vg_stream_read_blocks(void);
vg_status vg_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
vg_status vg_stream_read_config(const void* buf, size_t bytes, uint32_t* sink, int loads_in_flight,
                                int wgs_per_cu, void* stream);

/*
 * Debug: decode packed codes on the GPU into one byte per weight, codes[N, K] uint8 (0/1
 * for the 1-bit formats, 0..3 for the 2-bit ones), with the register decode the verify
 * GEMM itself runs for (format, x_dtype): the same extraction routine, fed the same masks
 * and magic constants the GEMM's launch builds (the 1-bit formats decode to bf16 operand
 * halves against VG_BF16 activations, to fp16 halves otherwise).  Each operand half holds
 * BETA + DELTA * code; the byte is (half - BETA) / DELTA with the same BETA the GEMM's
 * offset sums subtract, or 0xFF when the half is not exactly such a value, so tests can
 * compare the decoded codes with the packed words bit for bit ("Bonsai-27B-mlx-1bit" model
 * card, binary weight format: one bit per weight; the code-to-half construction:
 * "Ishizuki" README, credits).
 *   format   VG_FMT_SIGN1, VG_FMT_AFFINE2, VG_FMT_HAD2 or VG_FMT_AFFINE1; w holds [N, K/32]
 *            (1-bit) or [N, K/16] (2-bit) words, 16-byte aligned.
 *   x_dtype  VG_F16 or VG_BF16; VG_F32 -> VG_ERR_UNSUPPORTED (fp32 activations take the VALU
 *            kernel, which extracts each code with a shift and a mask instead).
 * Requires N >= 1 and K a positive multiple of 32 (1-bit) or 16 (2-bit).
 * vg_debug_unpack_sign1 and vg_debug_unpack_affine2 are this call with VG_F16.
 */
vg_status vg_debug_unpack(int format, int x_dtype, const uint32_t* w, int N, int K, uint8_t* codes,
                          void* stream);
vg_status vg_debug_unpack_sign1(const uint32_t* wbits, int N, int K, uint8_t* codes,
                                void* stream);
vg_status vg_debug_unpack_affine2(const uint32_t* wq, int N, int K, uint8_t* codes,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_GEMM_H */
