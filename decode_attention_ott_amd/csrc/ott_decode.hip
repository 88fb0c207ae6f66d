// Decoding stage of the OTT path for gfx950 (CDNA4, wave64).
//
// Method: "Accurate KV Cache Quantization with Outlier Tokens Tracing"
// (arXiv 2505.10938). [Blog] zijie-tian.site summary, section 3.3 and its
// flowchart: the query multiplies the quantized Keys, the fp16 window Keys and
// the outlier-pool Keys; the scores are concatenated under one softmax; the
// weights multiply the matching Values and the parts are summed ([Abs]
// sciencestack.ai, Figure 2 top). Here the concatenation is an online softmax:
// every wave keeps a running max m, a running sum l and an accumulator, and
// partial states merge as (m, l, acc) -> (M, sum l e^(m-M), sum acc e^(m-M)).
//
// A split is a byte-balanced slice of one (sequence, KV head)'s cache: a range
// of pages and a range of fp16 tokens (pool first, then the window). With one
// split the work-group writes the output; otherwise it writes its partial
// state and a second kernel merges the splits.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ott_decode_common.h"

namespace ott {
namespace {
using namespace dev;
using namespace dec;

// Dot of 16 2-bit codes (one dword, code i in bits 2i..2i+1) with 16 weights.
// A nibble whose two high bits are zero is the FP4 (E2M1) value code/2, so two
// masks turn the dword into 8 + 8 FP4 values and each byte converts to two
// floats in one instruction, so the result is half the true dot product.
__device__ __forceinline__ float dot16_codes(uint32_t w, const float4& c0, const float4& c1,
                                             const float4& c2, const float4& c3, float acc) {
  const uint32_t ev = w & 0x33333333u;         // codes 0 and 2 of every byte
  const uint32_t od = (w >> 2) & 0x33333333u;  // codes 1 and 3 of every byte
  f32x2 e, o;
  e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 0);
  acc = fmaf(c0.x, e.x, acc);
  acc = fmaf(c0.y, o.x, acc);
  acc = fmaf(c0.z, e.y, acc);
  acc = fmaf(c0.w, o.y, acc);
  e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 1);
  acc = fmaf(c1.x, e.x, acc);
  acc = fmaf(c1.y, o.x, acc);
  acc = fmaf(c1.z, e.y, acc);
  acc = fmaf(c1.w, o.y, acc);
  e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 2);
  acc = fmaf(c2.x, e.x, acc);
  acc = fmaf(c2.y, o.x, acc);
  acc = fmaf(c2.z, e.y, acc);
  acc = fmaf(c2.w, o.y, acc);
  e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 3);
  o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 3);
  acc = fmaf(c3.x, e.x, acc);
  acc = fmaf(c3.y, o.x, acc);
  acc = fmaf(c3.z, e.y, acc);
  acc = fmaf(c3.w, o.y, acc);
  return acc;
}

// Same for 16 codes against fp16 weights held as pairs per group of 4 slots:
// group g gives {(w[4g], w[4g+2]), (w[4g+1], w[4g+3])}, the order in which the
// FP4 -> f16 conversion returns codes (0,2) and (1,3) of a byte; pa holds
// groups 0 and 1 of the dword, pb groups 2 and 3. Half the true dot product.
__device__ __forceinline__ float dot16_codes_h(uint32_t w, const uint4& pa, const uint4& pb,
                                               float acc) {
  const uint32_t ev = w & 0x33333333u;
  const uint32_t od = (w >> 2) & 0x33333333u;
  acc = fdot2(pa.x, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 0)), acc);
  acc = fdot2(pa.y, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 0)), acc);
  acc = fdot2(pa.z, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 1)), acc);
  acc = fdot2(pa.w, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 1)), acc);
  acc = fdot2(pb.x, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 2)), acc);
  acc = fdot2(pb.y, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 2)), acc);
  acc = fdot2(pb.z, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 3)), acc);
  acc = fdot2(pb.w, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 3)), acc);
  return acc;
}

// Position of slot s in the pair layout read by dot16_codes_h.
__device__ __forceinline__ int pair_slot(int s) {
  return (s & ~3) | ((s & 1) << 1) | ((s >> 1) & 1);
}

// Online softmax state of one wave (scores in log2 units) while it walks
// quantized pages.
struct WaveState {
  float m;        // running max (wave-uniform)
  float l;        // this lane's share of the running sum of weights
  float vmin;     // this lane's share of sum p_t * min_t over quantized tokens
  // G = 128 (matrix-core pages): acc[0..3] digit-row sums of channel
  // 16(lane>>4) + (lane&15), acc[4..7] of that channel + 64, full units.
  // Other G: channel 16k + lane/4, slot quarter lane&3, half units.
  float acc[8];
};
__device__ __forceinline__ void rescale_q(WaveState& st, float m_new) {
  if (m_new == st.m) return;
  const float alpha = (st.m == -INFINITY) ? 0.f : exp2_fast(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  st.vmin *= alpha;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.acc[k] *= alpha;
}

// ---------------------------------------------------------------------------
// quantized pages
// ---------------------------------------------------------------------------
// Lane mapping inside a page (G tokens, d = 128 channels), quad = lanes 4i..4i+3:
//   K: pass k covers tokens 16k..16k+15; quad i takes token 16k+i, lane 4i+j
//      takes channels 32j..32j+31 (bytes 8j..8j+7 of the 32-byte code row).
//   V: pass k covers channels 16k..16k+15; quad i takes channel 16k+i, lane
//      4i+j takes slots (G/4)j..(G/4)j+G/4-1 (G/16 bytes of the channel row).
template <int G>
struct PageRegs {
  static constexpr int KP = G / 16;       // K passes
  static constexpr int VW = G / 64;       // V dwords per lane and channel (>= 1)
  uint2 kc[KP];
  uint32_t vc[8][VW];
  uint32_t vm[KP / 4];  // V (min, scale) of this lane's tokens 16(4i+j)+ti
  uint2 km;
};

// Loads in the order the page is consumed (K meta, K codes, V meta, V codes)
// so that each wait only covers what the next step needs.
template <int G>
__device__ __forceinline__ void load_page(PageRegs<G>& r, const uint8_t* __restrict__ pg,
                                          int lane) {
  constexpr int KP = PageRegs<G>::KP, VW = PageRegs<G>::VW;
  const int j = lane & 3, ti = lane >> 2;
  r.km = ld_nt2(pg + kmeta_off(G) + 8 * lane);
#pragma unroll
  for (int k = 0; k < KP; ++k) r.kc[k] = ld_nt2(pg + (16 * k + ti) * (D / 4) + 8 * j);
#pragma unroll
  for (int i = 0; i < KP / 4; ++i) r.vm[i] = ld_nt1(pg + vmeta_off(G) + 4 * (16 * (4 * i + j) + ti));
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint8_t* src = pg + vcode_off(G) + (16 * k + ti) * (G / 4) + j * (G / 16);
    if constexpr (VW == 4) {
      const uint4 t = ld_nt4(src);
      r.vc[k][0] = t.x; r.vc[k][1] = t.y; r.vc[k][2] = t.z; r.vc[k][3] = t.w;
    } else if constexpr (VW == 2) {
      const uint2 t = ld_nt2(src);
      r.vc[k][0] = t.x; r.vc[k][1] = t.y;
    } else {
      r.vc[k][0] = ld_nt1(src);
    }
  }
}

template <int G>
__device__ __forceinline__ void compute_page(const PageRegs<G>& r, int n_valid, float qs0,
                                             float qs1, float* qp, _Float16* ph, WaveState& st,
                                             int lane) {
  constexpr int KP = PageRegs<G>::KP, VW = PageRegs<G>::VW;
  const int j = lane & 3, ti = lane >> 2;
  // q'_c = q_c * scale_c (doubled for the code/2 view); bias = sum_c q_c * min_c
  const float qa = 2.0f * qs0 * hi_f(r.km.x), qb = 2.0f * qs1 * hi_f(r.km.y);
  const float bias = wave_sum(qs0 * lo_f(r.km.x) + qs1 * lo_f(r.km.y));
  *reinterpret_cast<float2*>(qp + 2 * lane) = make_float2(qa, qb);
  wave_lds_sync();

  float z[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) z[k] = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4* qv = reinterpret_cast<const float4*>(qp + 32 * j + 16 * h);
    const float4 c0 = qv[0], c1 = qv[1], c2 = qv[2], c3 = qv[3];
#pragma unroll
    for (int k = 0; k < KP; ++k)
      z[k] = dot16_codes(h ? r.kc[k].y : r.kc[k].x, c0, c1, c2, c3, z[k]);
  }
  // transpose-reduce inside the quad: afterwards lane j holds the full score
  // of tokens 16(4i+j)+ti, i = 0..KP/4-1
  constexpr int KT = KP / 4;
  float za[KP / 2];
#pragma unroll
  for (int i = 0; i < KP / 2; ++i) {
    const float keep = (j & 1) ? z[2 * i + 1] : z[2 * i];
    const float send = (j & 1) ? z[2 * i] : z[2 * i + 1];
    za[i] = keep + dpp<kQuadSwap1>(send);
  }
  float zt[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) {
    const float keep = (j & 2) ? za[2 * i + 1] : za[2 * i];
    const float send = (j & 2) ? za[2 * i] : za[2 * i + 1];
    zt[i] = keep + dpp<kQuadSwap2>(send) + bias;
  }
  if (n_valid < G) {  // only a page built while the pool was filling is short
#pragma unroll
    for (int i = 0; i < KT; ++i)
      if (16 * (4 * i + j) + ti >= n_valid) zt[i] = -INFINITY;
  }
  float mx = zt[0];
#pragma unroll
  for (int i = 1; i < KT; ++i) mx = fmaxf(mx, zt[i]);
  mx = wave_max(mx);
  if (mx == -INFINITY) return;  // a page without members
  rescale_q(st, fmaxf(st.m, mx));
#pragma unroll
  for (int i = 0; i < KT; ++i) {
    const float p = exp2_fast(zt[i] - st.m);
    st.l += p;
    st.vmin = fmaf(p, lo_f(r.vm[i]), st.vmin);
    // p' = p * scale_t stays below 2^16 (p <= 1, scale <= 2^16 / 3) in fp16
    ph[pair_slot(16 * (4 * i + j) + ti)] = _Float16(p * hi_f(r.vm[i]));
  }
  wave_lds_sync();
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    const uint4* pv = reinterpret_cast<const uint4*>(ph + j * (G / 4) + 16 * w);
    const uint4 pa = pv[0], pb = pv[1];
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[k] = dot16_codes_h(r.vc[k][w], pa, pb, st.acc[k]);
  }
  wave_lds_sync();
}

// ---------------------------------------------------------------------------
// quantized pages on the matrix cores (G = 128)
// ---------------------------------------------------------------------------
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
//
// Rows: A holds the 4 digit rows of the page four times (rows 4i..4i+3). The
// scale register packs one byte per replica; byte i is the real scale for
// replica i and 0 (2^-127) for the others, and tile T runs with op_sel T % 4.
// Tiles 0..3 accumulate into one result and 4..7 into another, so lane group g
// ends with exactly its own tiles g and g+4 (the masked products add at most
// 2^-110 in total).
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

// A operand: digit row (lane & 3) of a [4][128] byte block in logical k order
__device__ __forceinline__ i32x8 mx_a(const uint8_t* rows, int lane) {
  const uint8_t* r = rows + 128 * (lane & 3) + 16 * (lane >> 4);
  const uint4 lo = *reinterpret_cast<const uint4*>(r);
  const uint4 hi = *reinterpret_cast<const uint4*>(r + 64);
  i32x8 a;
  a[0] = int(lo.x); a[1] = int(lo.y); a[2] = int(lo.z); a[3] = int(lo.w);
  a[4] = int(hi.x); a[5] = int(hi.y); a[6] = int(hi.z); a[7] = int(hi.w);
  return a;
}

// Scale register: 2^(e-4-5k) for digit row k times 2 for the code/2 view, in
// the byte of the lane's replica.
__device__ __forceinline__ int mx_scale(int e, int lane) {
  return (124 - 5 * (lane & 3) + e) << (8 * ((lane >> 2) & 3));
}

__device__ __forceinline__ int mx_exp(float amax) {
  return max(__builtin_amdgcn_frexp_expf(amax), -100);
}

struct MxPage {
  uint2 kc[8];     // K tile T: token 16T + j, channel items 32g..32g+31
  uint2 vc[8];     // V tile C: channel 16C + j, slot items 32g..32g+31
  uint32_t km[2];  // K (min, scale) of the lane's channels c0 and c0 + 2
  uint32_t vm[2];  // V (min, scale) of the lane's slots 16g + j and 64 + 16g + j
};

__device__ __forceinline__ void mx_load(MxPage& r, const uint8_t* __restrict__ pg, int lane,
                                        int c0) {
  constexpr int G = 128;
  const int j = lane & 15, g = lane >> 4;
  r.km[0] = ld_nt1(pg + kmeta_off(G) + 4 * c0);
  r.km[1] = ld_nt1(pg + kmeta_off(G) + 4 * (c0 + 2));
#pragma unroll
  for (int T = 0; T < 8; ++T) r.kc[T] = ld_nt2(pg + (16 * T + j) * (D / 4) + 8 * g);
  r.vm[0] = ld_nt1(pg + vmeta_off(G) + 4 * (16 * g + j));
  r.vm[1] = ld_nt1(pg + vmeta_off(G) + 4 * (64 + 16 * g + j));
#pragma unroll
  for (int C = 0; C < 8; ++C) r.vc[C] = ld_nt2(pg + vcode_off(G) + (16 * C + j) * (G / 4) + 8 * g);
}

// One page. State layout: acc[0..3] are the digit-row partial sums of channel
// 16g + j, acc[4..7] those of channel 64 + 16g + j (full units); the lane's
// tokens are slots 16g + j and 64 + 16g + j.
__device__ __forceinline__ void mx_page(const MxPage& r, int n_valid, float qs0, float qs1,
                                        uint8_t* qa, uint8_t* pa, WaveState& st, int lane) {
  const int j = lane & 15, g = lane >> 4;
  // ---- scores: q'_c = q_c scale_c as digits, bias = sum_c q_c min_c
  const float qp0 = qs0 * hi_f(r.km[0]), qp1 = qs1 * hi_f(r.km[1]);
  const float bias = wave_sum(fmaf(qs0, lo_f(r.km[0]), qs1 * lo_f(r.km[1])));
  const int eq = mx_exp(wave_max(fmaxf(fabsf(qp0), fabsf(qp1))));
  {
    float d0[4], d1[4];
    mx_digits(qp0, eq, d0);
    mx_digits(qp1, eq, d1);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<uint16_t*>(qa + 128 * k + 2 * lane) =
          uint16_t(__builtin_amdgcn_cvt_pk_fp8_f32(d0[k], d1[k], 0, false));
  }
  wave_lds_sync();
  const i32x8 aq = mx_a(qa, lane);
  const int sq = mx_scale(eq, lane);
  f32x4v za = {0.f, 0.f, 0.f, 0.f}, zb = za;
  za = mx_mfma<0>(aq, mx_b(r.kc[0]), za, sq);
  zb = mx_mfma<0>(aq, mx_b(r.kc[4]), zb, sq);
  za = mx_mfma<1>(aq, mx_b(r.kc[1]), za, sq);
  zb = mx_mfma<1>(aq, mx_b(r.kc[5]), zb, sq);
  za = mx_mfma<2>(aq, mx_b(r.kc[2]), za, sq);
  zb = mx_mfma<2>(aq, mx_b(r.kc[6]), zb, sq);
  za = mx_mfma<3>(aq, mx_b(r.kc[3]), za, sq);
  zb = mx_mfma<3>(aq, mx_b(r.kc[7]), zb, sq);
  const int t0 = 16 * g + j;
  float z0 = bias + ((za[0] + za[1]) + (za[2] + za[3]));
  float z1 = bias + ((zb[0] + zb[1]) + (zb[2] + zb[3]));
  if (n_valid < 128) {  // only a page built while the pool was filling is short
    if (t0 >= n_valid) z0 = -INFINITY;
    if (t0 + 64 >= n_valid) z1 = -INFINITY;
  }
  const float mx = wave_max(fmaxf(z0, z1));
  if (mx == -INFINITY) return;  // a page without members
  rescale_q(st, fmaxf(st.m, mx));
  const float p0 = exp2_fast(z0 - st.m), p1 = exp2_fast(z1 - st.m);
  st.l += p0 + p1;
  st.vmin = fmaf(p0, lo_f(r.vm[0]), fmaf(p1, lo_f(r.vm[1]), st.vmin));
  // ---- values: p'_t = p_t scale_t as digits
  const float pp0 = p0 * hi_f(r.vm[0]), pp1 = p1 * hi_f(r.vm[1]);
  const int ep = mx_exp(wave_max(fmaxf(pp0, pp1)));
  {
    float d0[4], d1[4];
    mx_digits(pp0, ep, d0);
    mx_digits(pp1, ep, d1);
    const int kt = mx_k(t0);  // slot t0 + 64 sits at kt + 64
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(d0[k], d1[k], 0, false));
      pa[128 * k + kt] = uint8_t(w);
      pa[128 * k + kt + 64] = uint8_t(w >> 8);
    }
  }
  wave_lds_sync();
  const i32x8 ap = mx_a(pa, lane);
  const int sp = mx_scale(ep, lane);
  f32x4v va = {st.acc[0], st.acc[1], st.acc[2], st.acc[3]};
  f32x4v vb = {st.acc[4], st.acc[5], st.acc[6], st.acc[7]};
  va = mx_mfma<0>(ap, mx_b(r.vc[0]), va, sp);
  vb = mx_mfma<0>(ap, mx_b(r.vc[4]), vb, sp);
  va = mx_mfma<1>(ap, mx_b(r.vc[1]), va, sp);
  vb = mx_mfma<1>(ap, mx_b(r.vc[5]), vb, sp);
  va = mx_mfma<2>(ap, mx_b(r.vc[2]), va, sp);
  vb = mx_mfma<2>(ap, mx_b(r.vc[6]), vb, sp);
  va = mx_mfma<3>(ap, mx_b(r.vc[3]), va, sp);
  vb = mx_mfma<3>(ap, mx_b(r.vc[7]), vb, sp);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    st.acc[k] = va[k];
    st.acc[4 + k] = vb[k];
  }
  wave_lds_sync();
}

// ---------------------------------------------------------------------------
// the kernel (one query head per KV head)
// ---------------------------------------------------------------------------
// Work-group = 4 waves on one (sequence, head, split). The waves deal the
// split's pages round-robin, spread the fp16 chunks between their pages and
// merge their states in LDS.
struct alignas(16) WaveLds {
  float qp[D];          // q' of the current page
  _Float16 ph[256];     // p' of the current page, pair layout (G <= 256)
  float fin[4][D];      // fp16-path fold, then this wave's accumulator
};

// G <= 128 fits 128 VGPRs (4 waves per SIMD); G = 256 keeps two waves per SIMD.
template <int G>
__global__ __launch_bounds__(256, G <= 128 ? 4 : 2) void decode_kernel(Arena a, const __half* __restrict__ q,
                                                     __half* __restrict__ out, int S,
                                                     HeadOrder order) {
  __shared__ WaveLds lds_all[kWaves];
  __shared__ float mg_m[kWaves], mg_l[kWaves];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  WaveLds& L = lds_all[wave];
  const int s = blockIdx.x % S;
  const int bh = order.n ? int(order.bh[blockIdx.x]) : int(blockIdx.x / S);  // = b * H + h
  const int b = bh / a.Hkv;

  const int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  const int pc = min(a.P, a.G * nb);
  const Split sp = split_of(nb, pc + r_cnt, a.page_bytes, s, S);
  const int p1 = sp.p1, t1 = sp.t1;
  const int buf = nb & 1;
  const Fp16Src src{pool_k(a, buf, bh), pool_v(a, buf, bh), ring_k(a, bh), ring_v(a, bh), pc,
                    head, a.C};
  const float qscale = a.sm_scale * kLog2e;
  const uint8_t* pages = page_ptr(a, bh, 0);
  const int64_t PB = a.page_bytes;

  constexpr bool kMx = (G == 128);  // pages on the matrix cores
  const __half* qrow = q + size_t(bh) * D;
  const uint4 q8 = reinterpret_cast<const uint4*>(qrow)[lane & 15];
  // the lane's two channels: 2 lane, 2 lane + 1, or for the matrix-core pages
  // the channels of logical k = 2 lane, 2 lane + 1 (c0 and c0 + 2)
  const int c0 = kMx ? mx_item(2 * lane) : 2 * lane;
  const int c1 = kMx ? c0 + 2 : c0 + 1;
  const float qs0 = __half2float(qrow[c0]) * qscale, qs1 = __half2float(qrow[c1]) * qscale;
  WaveState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.vmin = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.acc[k] = 0.f;
  // fp16 chunks (memory-heavy) are spread between pages (compute-heavy),
  // staggered by wave, so the work-group always mixes the two
  int chunk = sp.t0 + wave * kF16Chunk;
  auto next_chunk = [&]() {
    Fp16State fs;
    fs.m = -INFINITY;
    fs.l = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) fs.acc[k] = 0.f;
    fp16_chunk(src, chunk, min(kF16Chunk, t1 - chunk), q8, qscale, fs, lane);
    chunk += kWaves * kF16Chunk;
    // fold (m, l, acc) of the chunk into the page state; acc changes layout
    // through LDS (channel 8*(lane&15)+e, row lane>>4 -> quad layout) and
    // enters in half units
    const float M = fmaxf(st.m, fs.m);
    rescale_q(st, M);
    const float af = (fs.m == -INFINITY) ? 0.f : exp2_fast(fs.m - M);
    st.l = fmaf(fs.l, af, st.l);
    const float ah = kMx ? af : 0.5f * af;
    float4* f = reinterpret_cast<float4*>(&L.fin[lane >> 4][8 * (lane & 15)]);
    f[0] = make_float4(fs.acc[0] * ah, fs.acc[1] * ah, fs.acc[2] * ah, fs.acc[3] * ah);
    f[1] = make_float4(fs.acc[4] * ah, fs.acc[5] * ah, fs.acc[6] * ah, fs.acc[7] * ah);
    wave_lds_sync();
    if constexpr (kMx) {
      const int ca = 16 * (lane >> 4) + (lane & 15);
      st.acc[0] += (L.fin[0][ca] + L.fin[1][ca]) + (L.fin[2][ca] + L.fin[3][ca]);
      st.acc[4] += (L.fin[0][ca + 64] + L.fin[1][ca + 64]) + (L.fin[2][ca + 64] + L.fin[3][ca + 64]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) st.acc[k] += L.fin[lane & 3][16 * k + (lane >> 2)];
    }
    wave_lds_sync();
  };
  int n = 0;
  for (int u = sp.p0 + wave; u < p1; u += kWaves, ++n) {
    prio_by_work_left((p1 - u + kWaves - 1) / kWaves);
    if constexpr (kMx) {
      MxPage pr;
      mx_load(pr, pages + size_t(u) * PB, lane, c0);
      mx_page(pr, page_nvalid(a.G, a.P, u), qs0, qs1, reinterpret_cast<uint8_t*>(L.qp),
              reinterpret_cast<uint8_t*>(L.ph), st, lane);
    } else {
      PageRegs<G> pr;
      load_page<G>(pr, pages + size_t(u) * PB, lane);
      compute_page<G>(pr, page_nvalid(a.G, a.P, u), qs0, qs1, L.qp, L.ph, st, lane);
    }
    if ((n & 3) == wave && chunk < t1) next_chunk();
  }
  while (chunk < t1) next_chunk();

  // this wave's state -> LDS in channel order (accumulator back to full units)
  const float l_tot = wave_sum(st.l);
  const float v_tot = wave_sum(st.vmin);
  if constexpr (kMx) {
    const int ca = 16 * (lane >> 4) + (lane & 15);
    L.fin[0][ca] = ((st.acc[0] + st.acc[1]) + (st.acc[2] + st.acc[3])) + v_tot;
    L.fin[0][ca + 64] = ((st.acc[4] + st.acc[5]) + (st.acc[6] + st.acc[7])) + v_tot;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[k] = quad_sum(st.acc[k]);
    if ((lane & 3) == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) L.fin[0][16 * k + (lane >> 2)] = fmaf(2.0f, st.acc[k], v_tot);
    }
  }
  if (lane == 0) {
    mg_m[wave] = st.m;
    mg_l[wave] = l_tot;
  }
  __syncthreads();
  // merge the 4 waves
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mg_m[w]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (mg_m[w] == -INFINITY) ? 0.f : exp2f(mg_m[w] - M);
      Ls = fmaf(mg_l[w], f, Ls);
      A = fmaf(lds_all[w].fin[0][c], f, A);
    }
    if (S == 1) {
      out[size_t(bh) * D + c] = __float2half_rn(A / Ls);
    } else {
      float* part = partial_ptr(a, b, bh % a.Hq, s);
      part[2 + c] = A;
      if (c == 0) {
        part[0] = M;
        part[1] = Ls;
      }
    }
  }
}

// Merge of S split partial states per (sequence, query head): the partials
// are read 16 at a time with all loads in flight, then merged online
// (M, L, A) <- (max, L e^(M-M') + sum l e^(m-M'), A e^(M-M') + sum acc e^(m-M')).
__global__ __launch_bounds__(D) void combine_kernel(Arena a, __half* __restrict__ out, int S) {
  constexpr int kChunk = 16;
  const int bq = blockIdx.x;  // b * Hq + qh
  const int c = threadIdx.x;
  const float* part = reinterpret_cast<const float*>(a.base + a.off_partials) +
                      size_t(bq) * a.max_splits * (2 + D);
  float M = -INFINITY, Ls = 0.f, A = 0.f;
  for (int i0 = 0; i0 < S; i0 += kChunk) {
    float m[kChunk], l[kChunk], v[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const bool ok = i0 + k < S;
      const float* p = part + size_t(ok ? i0 + k : 0) * (2 + D);
      m[k] = ok ? p[0] : -INFINITY;
      l[k] = p[1];
      v[k] = p[2 + c];
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) Mc = fmaxf(Mc, m[k]);
    if (Mc == -INFINITY) continue;
    const float f0 = (M == -INFINITY) ? 0.f : exp2f(M - Mc);
    Ls *= f0;
    A *= f0;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float f = (m[k] == -INFINITY) ? 0.f : exp2f(m[k] - Mc);
      Ls = fmaf(l[k], f, Ls);
      A = fmaf(v[k], f, A);
    }
    M = Mc;
  }
  out[size_t(bq) * D + c] = __float2half_rn(A / Ls);
}

}  // namespace

int decode_wgs_per_cu(const Arena& a) {
  if (a.Hq != a.Hkv) return decode_gqa_wgs_per_cu(a);
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (a.G) {
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<64>, 64 * kWaves, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<128>, 64 * kWaves, 0); break;
    case 256: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<256>, 64 * kWaves, 0); break;
    default: break;
  }
  return e == hipSuccess ? n : 0;
}

hipError_t launch_decode(const Arena& a, const void* q, void* out, int S, const HeadOrder& order,
                         hipStream_t s) {
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  hipError_t e;
  if (a.Hq != a.Hkv) {
    e = launch_decode_gqa(a, q, out, S, order, s);
  } else {
    const dim3 grid(unsigned(a.B) * a.Hkv * S);
    switch (a.G) {
      case 64: hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order); break;
      case 128: hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order); break;
      case 256: hipLaunchKernelGGL(decode_kernel<256>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(a.B) * a.Hq), dim3(D), 0, s, a, oh, S);
  return hipGetLastError();
}

}  // namespace ott
