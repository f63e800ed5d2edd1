// vg_device.h -- device helpers of the verify GEMM (gfx950): packed-code extraction.
//
// A packed word is decoded straight into fp16 MFMA operand registers, two codes per
// register, with one bitwise AND-OR per register and no conversion instruction.  This is
// the same idea as the exact code-to-half trick with 0x6400 ("Ishizuki" README, Credits:
// codes turned into exact halves), generalised so every bit position of the word can be
// used in place:
//
//   reg = (word & mask_p) | magic_p     with mask_p selecting bit(s) p and p+16,
//
// where magic_p is an fp16 pair whose exponent is chosen per position p so that setting
// the code's bits adds exactly  code * DELTA  to the magic's value BETA_p, with the same
// DELTA for every position.  An operand register therefore holds  BETA + DELTA * code  in
// each half, exactly.  The constant part  sum_k a_k * BETA_k  is removed per (row, group)
// with a correction computed once per workgroup from the activations, so the codes are
// never shifted down or converted one by one.
//
// Register pairing: the two halves of a register hold the codes at bits p (low half) and
// p+16 (high half) of the same shifted word, i.e. K indices k and k+16 (1-bit format) or
// k and k+8 (2-bit format) of the word's window.  The activation operand is laid out to
// match (see the staging code in vg_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vg {

// AFFINE1: MLX's 1-bit affine codes (w = bit * s + b, one scale and bias per 128 weights),
// decoded like the sign bits and finished like the 2-bit affine format.
enum Format : int { SIGN1 = 0, AFFINE2 = 1, HAD2 = 2, AFFINE1 = 3 };
__host__ __device__ constexpr bool fmt_one_bit(int fmt) { return fmt == SIGN1 || fmt == AFFINE1; }

// ---- 1-bit sign format: 16 registers per 32-bit word ---------------------------------
// Register b0 (0..15) holds the bits b0 and b0+16 of the word, taken at position p of a
// shifted copy:  b0 0..4 -> (w << 5) at p = b0+5;  b0 5..10 -> w at p = b0;
// b0 11..15 -> (w >> 6) at p = b0-6.  Positions 5..9 are mantissa bits (magic exponent
// 26-p, BETA = 2^(11-p)); position 10 is the exponent's lowest bit (magic 2.0 -> 4.0).
// DELTA = 2 everywhere, so a register half equals BETA_b0 + 2 * bit.
__host__ __device__ constexpr int sign1_pos(int b0) { return b0 < 5 ? b0 + 5 : (b0 <= 10 ? b0 : b0 - 6); }
__host__ __device__ constexpr int sign1_src(int b0) { return b0 < 5 ? 1 : (b0 <= 10 ? 0 : 2); }  // 0: w, 1: w<<5, 2: w>>6
__host__ __device__ constexpr uint32_t half_magic_sign1(int p) {
  return p == 10 ? 0x4000u : (uint32_t)(26 - p) << 10;
}
__host__ __device__ constexpr float sign1_beta(int b0) {
  return sign1_pos(b0) == 10 ? 2.0f : (float)(1 << (11 - sign1_pos(b0)));
}
constexpr float SIGN1_DELTA = 2.0f;

// ---- 1-bit codes against bf16 activations: bf16 operand halves ------------------------
// With bf16 activations the MFMA takes bf16 on both sides, so the codes decode to bf16
// (7 stored mantissa bits).  Register b0 (0..15) holds the bits b0 and b0+16 of the word,
// taken at position p = b0 & 7 of w (b0 < 8) or of w >> 8 (b0 >= 8).  Positions 0..6 are
// mantissa bits (magic exponent 135-p, BETA = 2^(8-p)); position 7 is the exponent's
// lowest bit (magic 2.0 -> 4.0).  DELTA = 2 again, and every BETA + 2 is a bf16 value.
__host__ __device__ constexpr uint32_t bf16_magic_sign1(int p) {
  return p == 7 ? 0x4000u : (uint32_t)(135 - p) << 7;
}
__host__ __device__ constexpr float sign1_beta_bf16(int b0) {
  return (b0 & 7) == 7 ? 2.0f : (float)(1 << (8 - (b0 & 7)));
}

// ---- 2-bit affine format: 8 registers per 32-bit word ---------------------------------
// Register j (0..7) holds codes j and j+8 (bits 2j.. and 2j+16..), taken at position p of
// a shifted copy:  j 0,1 -> (w << 6) at p = 2j+6;  j 2..4 -> w at p = 2j;
// j 5..7 -> (w >> 6) at p = 2j-6.  Magic exponent 25-p, BETA = 2^(10-p), DELTA = 1, so a
// register half equals BETA_j + code.
__host__ __device__ constexpr int affine2_pos(int j) { return j < 2 ? 2 * j + 6 : (j <= 4 ? 2 * j : 2 * j - 6); }
__host__ __device__ constexpr int affine2_src(int j) { return j < 2 ? 1 : (j <= 4 ? 0 : 2); }  // 0: w, 1: w<<6, 2: w>>6
__host__ __device__ constexpr uint32_t half_magic_affine2(int p) { return (uint32_t)(25 - p) << 10; }
__host__ __device__ constexpr float affine2_beta(int j) { return (float)(1 << (10 - affine2_pos(j))); }
constexpr float AFFINE2_DELTA = 1.0f;

}  // namespace vg
