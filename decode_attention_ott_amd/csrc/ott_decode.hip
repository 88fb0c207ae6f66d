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

#include "ott_device.h"

namespace ott {
namespace {
using namespace dev;

constexpr int kWaves = 4;           // waves (work items) per work-group
constexpr int kFp16TokenBytes = 4 * D;  // K + V bytes of one fp16 token

// ---------------------------------------------------------------------------
// cross-lane helpers (DPP inside 16-lane rows, permlane swaps across rows)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// every lane of a 16-lane row receives the row's sum / max
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return x;
}
// combine each lane with its partner row (lane ^ 16) / partner half (lane ^ 32)
__device__ __forceinline__ f32x2 swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return f32x2{__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1]))};
}
__device__ __forceinline__ f32x2 swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return f32x2{__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1]))};
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum(x);
  f32x2 p = swap16(x);
  x = p.x + p.y;
  p = swap32(x);
  return p.x + p.y;
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max(x);
  f32x2 p = swap16(x);
  x = fmaxf(p.x, p.y);
  p = swap32(x);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float pair_sum(float x) { return x + dpp<kQuadSwap1>(x); }

// Orders this wave's LDS writes before its later LDS reads. A wave's LDS
// instructions execute in issue order, so only the compiler must be kept from
// moving them; a memory fence here would also wait for every outstanding
// global load (the next page's codes included).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float lo_f(uint32_t w) {
  return __half2float(__ushort_as_half(uint16_t(w & 0xffffu)));
}
__device__ __forceinline__ float hi_f(uint32_t w) {
  return __half2float(__ushort_as_half(uint16_t(w >> 16)));
}
__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// Dot of 16 2-bit codes (one dword, code i in bits 2i..2i+1) with 16 weights.
// A nibble whose two high bits are zero is the FP4 (E2M1) value code/2, so two
// masks turn the dword into 8 + 8 FP4 values and each byte converts to two
// floats in one instruction. Weights must be pre-doubled.
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
// groups 0 and 1 of the dword, pb groups 2 and 3. Weights pre-doubled.
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

__device__ __forceinline__ uint32_t dw(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Streaming (non-temporal) loads: each cached byte is read once per decode.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_nt2(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_nt4(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt1(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p));
}

// 2^x with one v_exp_f32 (denormal results flush to zero: such softmax
// weights are below 2^-126 of the running maximum and do not matter).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax state of one wave (scores in log2 units) while it walks
// quantized pages.
struct WaveState {
  float m;        // running max (wave-uniform)
  float l;        // this lane's share of the running sum of weights
  float vmin;     // this lane's share of sum p_t * min_t over quantized tokens
  float acc[8];   // channel 16k + lane/4, slot quarter lane&3
};
// The same while it walks fp16 tokens (done first, then folded into WaveState).
struct Fp16State {
  float m;
  float l;
  float acc[8];   // channels 8*(lane&15) .. +7, tokens of row lane>>4
};

template <int N, typename St>
__device__ __forceinline__ void rescale(St& st, float m_new) {
  if (m_new == st.m) return;  // wave-uniform: the running max did not move
  const float alpha = (st.m == -INFINITY) ? 0.f : exp2_fast(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int k = 0; k < N; ++k) st.acc[k] *= alpha;
}
__device__ __forceinline__ void rescale_q(WaveState& st, float m_new) {
  if (m_new == st.m) return;
  const float alpha = (st.m == -INFINITY) ? 0.f : exp2_fast(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  st.vmin *= alpha;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.acc[k] *= alpha;
}

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  return x;
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
    ph[pair_slot(16 * (4 * i + j) + ti)] = _Float16(2.0f * p * hi_f(r.vm[i]));
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
// fp16 tokens: the pool (index i < pc) then the window (ring slot (head+i-pc)%C)
// ---------------------------------------------------------------------------
// 16 lanes share one token (lane&15 takes channels 8*(lane&15)..+7), so every
// load instruction reads 4 whole 256-byte rows. Scores reduce inside the row
// with DPP; the row then holds the token's weight for its V accumulation.
struct Fp16Src {
  const __half* pk;
  const __half* pv;
  const __half* rk;
  const __half* rv;
  int pc, head, C;
  __device__ __forceinline__ size_t row(int i) const {
    if (i < pc) return size_t(i) * D;
    const int x = head + i - pc;  // < 2C: head < C and i - pc < r_cnt <= C
    return size_t(x >= C ? x - C : x) * D;
  }
  __device__ __forceinline__ const __half* k(int i) const { return (i < pc ? pk : rk) + row(i); }
  __device__ __forceinline__ const __half* v(int i) const { return (i < pc ? pv : rv) + row(i); }
};

constexpr int kF16Pass = 4;                 // 4 tokens per pass
constexpr int kF16Chunk = 4 * kF16Pass;     // tokens per chunk

__device__ __forceinline__ void fp16_chunk(const Fp16Src& src, int base, int cnt, const uint4& q8,
                                           float qscale, Fp16State& st, int lane) {
  const int rw = lane >> 4, c8 = lane & 15;
  float z[kF16Pass];
  uint4 kv[kF16Pass], vv[kF16Pass];
  // rows past the chunk read the chunk's last token (in bounds); their
  // weights are forced to zero below. K and V rows are requested together.
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) kv[p] = ld_nt4(src.k(base + min(4 * p + rw, cnt - 1)) + 8 * c8);
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) vv[p] = ld_nt4(src.v(base + min(4 * p + rw, cnt - 1)) + 8 * c8);
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) {
    float acc = fdot2(kv[p].x, q8.x, 0.f);
    acc = fdot2(kv[p].y, q8.y, acc);
    acc = fdot2(kv[p].z, q8.z, acc);
    acc = fdot2(kv[p].w, q8.w, acc);
    z[p] = (4 * p + rw < cnt) ? row_sum(acc) * qscale : -INFINITY;
    mx = fmaxf(mx, z[p]);
  }
  {
    f32x2 pm = swap16(mx);
    mx = fmaxf(pm.x, pm.y);
    pm = swap32(mx);
    mx = fmaxf(pm.x, pm.y);
  }
  rescale<8>(st, fmaxf(st.m, mx));
  float lsum = 0.f;
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) {
    const float w = exp2_fast(z[p] - st.m);
    lsum += w;
    st.acc[0] = fmaf(w, lo_f(vv[p].x), st.acc[0]);
    st.acc[1] = fmaf(w, hi_f(vv[p].x), st.acc[1]);
    st.acc[2] = fmaf(w, lo_f(vv[p].y), st.acc[2]);
    st.acc[3] = fmaf(w, hi_f(vv[p].y), st.acc[3]);
    st.acc[4] = fmaf(w, lo_f(vv[p].z), st.acc[4]);
    st.acc[5] = fmaf(w, hi_f(vv[p].z), st.acc[5]);
    st.acc[6] = fmaf(w, lo_f(vv[p].w), st.acc[6]);
    st.acc[7] = fmaf(w, hi_f(vv[p].w), st.acc[7]);
  }
  if (c8 == 0) st.l += lsum;  // each row's tokens counted once
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// Work-group = 4 waves on one (sequence, KV head, split). With one query head
// per KV head the 4 waves share the split (pages and 32-token chunks dealt
// round-robin) and merge in LDS; with a query-head group every wave takes its
// own query head(s) over the whole split.
struct alignas(16) WaveLds {
  float qp[D];          // q' of the current page
  _Float16 ph[256];     // p' of the current page, pair layout (G <= 256)
  float fin[4][D];      // fp16-path fold, then this wave's accumulator
};

// G <= 128 fits 128 VGPRs (4 waves per SIMD); G = 256 keeps two waves per SIMD.
template <int G>
__global__ __launch_bounds__(256, G <= 128 ? 4 : 2) void decode_kernel(Arena a, const __half* __restrict__ q,
                                                     __half* __restrict__ out, int S) {
  __shared__ WaveLds lds_all[kWaves];
  __shared__ float mg_m[kWaves], mg_l[kWaves];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  WaveLds& L = lds_all[wave];
  const int NQ = a.Hq / a.Hkv;
  const int s = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int b = bh / a.Hkv, h = bh % a.Hkv;

  const int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  const int pc = min(a.P, a.G * nb);
  const int n16 = pc + r_cnt;
  // byte-balanced split: pages first, then fp16 tokens
  const int64_t PB = a.page_bytes;
  const int64_t W = nb * PB + int64_t(n16) * kFp16TokenBytes;
  const int64_t lo = int64_t(s) * W / S, hi = int64_t(s + 1) * W / S;
  auto first_page = [&](int64_t x) { return int(min<int64_t>(nb, (x + PB - 1) / PB)); };
  auto first_tok = [&](int64_t x) {
    const int64_t r = x - nb * PB;
    return r <= 0 ? 0 : int(min<int64_t>(n16, (r + kFp16TokenBytes - 1) / kFp16TokenBytes));
  };
  const int p0 = first_page(lo), p1 = first_page(hi);
  const int t0 = first_tok(lo), t1 = first_tok(hi);
  const int buf = nb & 1;
  const Fp16Src src{pool_k(a, buf, bh), pool_v(a, buf, bh), ring_k(a, bh), ring_v(a, bh), pc,
                    head, a.C};
  const float qscale = a.sm_scale * kLog2e;
  const uint8_t* pages = page_ptr(a, bh, 0);

  const int wph = NQ >= kWaves ? 1 : kWaves / NQ;  // waves per query head
  const int hpr = kWaves / wph;                    // query heads per round
  const int rounds = (NQ + hpr - 1) / hpr;
  for (int r = 0; r < rounds; ++r) {
    const int qi = r * hpr + wave / wph;
    const int stripe = wave % wph;
    if (qi < NQ) {
      const int qh = h * NQ + qi;
      const __half* qrow = q + (size_t(b) * a.Hq + qh) * D;
      const uint32_t q2 = reinterpret_cast<const uint32_t*>(qrow)[lane];
      const uint4 q8 = reinterpret_cast<const uint4*>(qrow)[lane & 15];
      const float qs0 = lo_f(q2) * qscale, qs1 = hi_f(q2) * qscale;
      WaveState st;
      st.m = -INFINITY;
      st.l = 0.f;
      st.vmin = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) st.acc[k] = 0.f;
      // fp16 chunks (memory-heavy) are spread between pages (compute-heavy),
      // staggered by wave, so the work-group always mixes the two
      int chunk = t0 + stripe * kF16Chunk;
      auto next_chunk = [&]() {
        Fp16State fs;
        fs.m = -INFINITY;
        fs.l = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) fs.acc[k] = 0.f;
        fp16_chunk(src, chunk, min(kF16Chunk, t1 - chunk), q8, qscale, fs, lane);
        chunk += wph * kF16Chunk;
        // fold (m, l, acc) of the chunk into the page state; acc changes
        // layout through LDS (channel 8*(lane&15)+e, row lane>>4 -> quad layout)
        const float M = fmaxf(st.m, fs.m);
        rescale_q(st, M);
        const float af = (fs.m == -INFINITY) ? 0.f : exp2_fast(fs.m - M);
        st.l = fmaf(fs.l, af, st.l);
        float4* f = reinterpret_cast<float4*>(&L.fin[lane >> 4][8 * (lane & 15)]);
        f[0] = make_float4(fs.acc[0] * af, fs.acc[1] * af, fs.acc[2] * af, fs.acc[3] * af);
        f[1] = make_float4(fs.acc[4] * af, fs.acc[5] * af, fs.acc[6] * af, fs.acc[7] * af);
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < 8; ++k) st.acc[k] += L.fin[lane & 3][16 * k + (lane >> 2)];
        wave_lds_sync();
      };
      int n = 0;
      for (int u = p0 + stripe; u < p1; u += wph, ++n) {
        PageRegs<G> pr;
        load_page<G>(pr, pages + size_t(u) * PB, lane);
        compute_page<G>(pr, page_nvalid(a.G, a.P, u), qs0, qs1, L.qp, L.ph, st, lane);
        if ((n & 3) == (stripe & 3) && chunk < t1) next_chunk();
      }
      while (chunk < t1) next_chunk();

      // this wave's state -> LDS in channel order
      const float l_tot = wave_sum(st.l);
      const float v_tot = wave_sum(st.vmin);
#pragma unroll
      for (int k = 0; k < 8; ++k) st.acc[k] = quad_sum(st.acc[k]);
      if ((lane & 3) == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) L.fin[0][16 * k + (lane >> 2)] = st.acc[k] + v_tot;
      }
      if (lane == 0) {
        mg_m[wave] = st.m;
        mg_l[wave] = l_tot;
      }
    }
    __syncthreads();
    // merge the waves of each query head of this round
    for (int jx = threadIdx.x; jx < hpr * D; jx += blockDim.x) {
      const int hr = jx / D, c = jx % D;
      const int qi2 = r * hpr + hr;
      if (qi2 >= NQ) continue;
      float M = -INFINITY;
      for (int w = hr * wph; w < (hr + 1) * wph; ++w) M = fmaxf(M, mg_m[w]);
      float Ls = 0.f, A = 0.f;
      for (int w = hr * wph; w < (hr + 1) * wph; ++w) {
        const float f = (mg_m[w] == -INFINITY) ? 0.f : exp2f(mg_m[w] - M);
        const float aw = lds_all[w].fin[0][c];
        Ls = fmaf(mg_l[w], f, Ls);
        A = fmaf(aw, f, A);
      }
      const int qh = h * NQ + qi2;
      if (S == 1) {
        out[(size_t(b) * a.Hq + qh) * D + c] = __float2half_rn(A / Ls);
      } else {
        float* part = reinterpret_cast<float*>(a.base + a.off_partials) +
                      ((size_t(b) * a.Hq + qh) * a.max_splits + s) * (2 + D);
        part[2 + c] = A;
        if (c == 0) {
          part[0] = M;
          part[1] = Ls;
        }
      }
    }
    __syncthreads();
  }
}

// Merge of S split partial states per (sequence, query head).
__global__ __launch_bounds__(D) void combine_kernel(Arena a, __half* __restrict__ out, int S) {
  const int bq = blockIdx.x;  // b * Hq + qh
  const int c = threadIdx.x;
  const float* part = reinterpret_cast<const float*>(a.base + a.off_partials) +
                      size_t(bq) * a.max_splits * (2 + D);
  float M = -INFINITY;
  for (int i = 0; i < S; ++i) M = fmaxf(M, part[i * (2 + D)]);
  float Ls = 0.f, A = 0.f;
  for (int i = 0; i < S; ++i) {
    const float m = part[i * (2 + D)];
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    Ls = fmaf(part[i * (2 + D) + 1], f, Ls);
    A = fmaf(part[i * (2 + D) + 2 + c], f, A);
  }
  out[size_t(bq) * D + c] = __float2half_rn(A / Ls);
}

}  // namespace

hipError_t launch_decode(const Arena& a, const void* q, void* out, int S, hipStream_t s) {
  const dim3 grid(unsigned(a.B) * a.Hkv * S);
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  switch (a.G) {
    case 64: hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S); break;
    case 128: hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S); break;
    case 256: hipLaunchKernelGGL(decode_kernel<256>, grid, dim3(64 * kWaves), 0, s, a, qh, oh, S); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(a.B) * a.Hq), dim3(D), 0, s, a, oh, S);
  return hipGetLastError();
}

}  // namespace ott
