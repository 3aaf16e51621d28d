// Device building blocks shared by the MXFP4 kernels (gfx950 only).
//
// quant32: one 32-element MXFP4 block quantised in registers -- the on-chip
// quantisation step of the fused plan in kernelbot amd-mxfp4-mm submission
// 517169 (module docstring: abs-max per 32, E8M0 scale, pack to fp4x2), with
// the OCP MX shared-exponent rule and round-to-nearest-even.
//
// mfma_fp4: the CDNA4 scaled matrix instruction V_MFMA_SCALE_F32_16X16X128_F8F6F4
// with both operands in E2M1 -- the block-scaled dot of the fused plan. Operand
// layout for lane l (0..63) of a wave:
//   A: row l%16 of the 16x128 tile, elements k = 32*(l/16) .. +31, 16 bytes,
//      first element in the low nibble of the first byte;
//   B: column (= row of B[N,K]) l%16, the same k range;
//   scale operands: one E8M0 byte per lane for exactly that (row, 32-k chunk),
//      chosen from the 32-bit register by the byte-select immediate;
//   result: lane l, register r holds D[4*(l/16) + r][l%16].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// E2M1 operand format code of the f8f6f4 matrix instructions.
constexpr int kFmtFp4 = 4;
// E8M0 byte of the neutral scale 2^0.
constexpr uint32_t kScaleOne = 127u;

// E8M0 byte from the bf16 bit pattern of a block's amax (a non-negative finite
// value): floor(log2 amax) - 2 in biased form is (exponent field - 2), clamped
// at 0 (= 2^-127), which also covers subnormal amax (exponent field 0); an
// all-zero block gets 127. The upper clamp (byte 254) is unreachable for bf16.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;
  return amax_bits == 0u ? kScaleOne : (e > 2u ? e - 2u : 0u);
}

__device__ __forceinline__ v2u16 abs_pair(uint32_t w) {
  return __builtin_bit_cast(v2u16, w & 0x7fff7fffu);
}

// The max of the 15-bit magnitude fields of 32 bf16 values held two per dword.
// For non-negative finite bf16 the bit pattern orders like the value, so this is
// the bit pattern of amax, exactly.
__device__ __forceinline__ uint32_t amax_bits32(const uint32_t (&w)[16]) {
  v2u16 m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = __builtin_elementwise_max(abs_pair(w[2 * i]), abs_pair(w[2 * i + 1]));
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = __builtin_elementwise_max(m[2 * i], m[2 * i + 1]);
  m[0] = __builtin_elementwise_max(m[0], m[1]);
  m[2] = __builtin_elementwise_max(m[2], m[3]);
  m[0] = __builtin_elementwise_max(m[0], m[2]);
  return m[0][0] > m[0][1] ? m[0][0] : m[0][1];
}

// Quantise 32 bf16 (w[i] holds elements 2i in bits 0-15 and 2i+1 in bits 16-31)
// to 32 E2M1 codes (q[d] byte j = elements 8d+2j (low nibble), 8d+2j+1) and the
// block's E8M0 byte. The hardware convert divides by the scale given as a float
// whose exponent field is the E8M0 byte, rounds to nearest even, saturates at
// +-6 and keeps the sign of zero; that matches the OCP rule for every finite bf16
// input and every scale byte 0..254 (checked exhaustively on gfx950).
__device__ __forceinline__ void quant32(const uint32_t (&w)[16], uint32_t (&q)[4], uint32_t& sbyte) {
  sbyte = e8m0_from_amax_bits(amax_bits32(w));
  const float scale = __builtin_bit_cast(float, sbyte << 23);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[4 * d + 0]), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[4 * d + 1]), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[4 * d + 2]), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[4 * d + 3]), scale, 3);
    q[d] = r;
  }
}

// Quantise the 8 bf16 held by this lane (w[i]: elements 2i, 2i+1) as one quarter
// of a 32-element MXFP4 block spread over the 4 lanes of an aligned lane quad
// (lanes 4a .. 4a+3, all active). The block's amax is the max of the four lanes'
// maxima, combined with two quad-permute DPP steps, so every lane of the quad
// derives the same E8M0 byte. Returns this lane's 8 E2M1 codes (element 2i in
// the low nibble of byte i). For use inside the GEMM, where the byte only scales
// the matrix instruction's product: an all-zero block gets byte 0 instead of
// e8m0_from_amax_bits' 127 (its codes are zero, so the product is zero under
// any finite scale), which leaves a saturating subtract as the whole rule.
// EXACT_ZERO: give an all-zero block the E8M0 byte 127 of the full rule
// (e8m0_from_amax_bits), for callers that store the scale bytes.
template <bool EXACT_ZERO = false>
__device__ __forceinline__ uint32_t quant8_quad(const uint32_t (&w)[4], uint32_t& sbyte) {
  const v2u16 m2 = __builtin_elementwise_max(__builtin_elementwise_max(abs_pair(w[0]), abs_pair(w[1])),
                                             __builtin_elementwise_max(abs_pair(w[2]), abs_pair(w[3])));
  uint32_t a = m2[0] > m2[1] ? m2[0] : m2[1];
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  a = a > o ? a : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  a = a > o ? a : o;
  sbyte = EXACT_ZERO ? e8m0_from_amax_bits(a) : __builtin_elementwise_sub_sat(a >> 7, 2u);  // max(e - 2, 0)
  const float scale = __builtin_bit_cast(float, sbyte << 23);
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[3]), scale, 3);
  return r;
}

// acc += (A * 2^(sa-127)) . (B * 2^(sb-127))^T over one 16x16x128 step.
// SA/SB select which byte of the 32-bit scale registers is used.
template <int SA = 0, int SB = 0>
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f acc, uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, kFmtFp4, kFmtFp4, SA, (int)sa, SB,
                                                          (int)sb);
}

// acc += A . B^T over one 32x32x64 step (V_MFMA_SCALE_F32_32X32X64_F8F6F4, E2M1
// operands). Lane l holds row (column of B) l%32 and k-chunk l/32 of its 32x64
// operand plus that block's scale byte; result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
template <int SA = 0, int SB = 0>
__device__ __forceinline__ v16f mfma32_fp4(const uint4& a, const uint4& b, v16f acc, uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, kFmtFp4, kFmtFp4, SA, (int)sa, SB,
                                                         (int)sb);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest even: the gfx950
// packed convert.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf));
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace mx
