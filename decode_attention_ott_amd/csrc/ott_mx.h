#pragma once
// Helpers for page products on the gfx950 fp8 x fp4 matrix cores, shared by
// the decode kernels.
//
// Both page products run on v_mfma_scale_f32_16x16x128_f8f6f4 with A = fp8
// (E4M3) weight digits and B = the page's 2-bit codes read as FP4 (E2M1): with
// its two high bits cleared, a code nibble is the FP4 value code/2, so a code
// dword becomes two B dwords with two masks and no conversion.
//
// Operand layout of that instruction (lane l, j = l & 15, g = l >> 4):
//   B: column j; byte-nibble n of dword w is logical k = 32g + 8w + n.
//   A: row j; byte b is logical k = 16g + (b & 15) + 64 (b >> 4).
//   D: column j, rows 4g..4g+3 in the four result registers.
//   The E8M0 scale of A row r for k-block kb is the op_sel byte of lane r+16kb.
// The lane's B chunk is 8 code bytes (32 items, item 4i+h at bits 2h of byte
// i); after the masks, logical k holds item mx_item(k) of the page row.
//
// Exactness: the matrix core sums one instruction's products with a limited
// number of bits below the largest, so every weight is split into 4
// fixed-point digits in [-16, 16] relative to one power of two 2^e per page
// and kind (digit k has step 2^(e-4-5k)). A row of digits times code/2 gives
// products on one grid of half-steps, at most 24 steps each, whose sums are
// exact; the step enters as the row's E8M0 scale. 4 digits keep 19 bits of the
// largest weight of the page.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ott {
namespace dec {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr uint32_t kCodeMask = 0x33333333u;

// item of logical k (channel for K, slot for V), and its inverse
__device__ __forceinline__ int mx_item(int k) {
  return (k & ~31) | (k & 16) | ((k >> 3) & 1) | ((k & 7) << 1);
}
__device__ __forceinline__ int mx_k(int t) {
  return (t & ~31) | (t & 16) | ((t & 1) << 3) | ((t & 15) >> 1);
}

__device__ __forceinline__ i32x8 mx_b(uint2 c) {
  i32x8 b;
  b[0] = int(c.x & kCodeMask);
  b[1] = int((c.x >> 2) & kCodeMask);
  b[2] = int(c.y & kCodeMask);
  b[3] = int((c.y >> 2) & kCodeMask);
  b[4] = 0;
  b[5] = 0;
  b[6] = 0;
  b[7] = 0;
  return b;
}

template <int SEL>
__device__ __forceinline__ f32x4v mx_mfma(const i32x8& a, const i32x8& b, const f32x4v& c, int sc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0 /* A: fp8 e4m3 */,
                                                          4 /* B: fp4 e2m1 */, SEL, sc, 0, 127);
}

// x = sum_k d[k] 2^(e-4-5k) + r with |r| <= 2^(e-20), given |x| < 2^e
__device__ __forceinline__ void mx_digits(float x, int e, float (&d)[4]) {
  float r = __builtin_amdgcn_ldexpf(x, 4 - e);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    d[k] = __builtin_rintf(r);
    r = (r - d[k]) * 32.0f;
  }
}

// exponent e with |x| < 2^e for the largest |x| of a row (clamped so that the
// digit scales stay inside the E8M0 range)
__device__ __forceinline__ int mx_exp(float amax) {
  return max(__builtin_amdgcn_frexp_expf(amax), -100);
}

}  // namespace dec
}  // namespace ott
