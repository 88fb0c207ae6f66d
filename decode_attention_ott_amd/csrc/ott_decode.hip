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
  float acc[8];   // channel 16k + lane/4, slot quarter lane&3; half units
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

  const __half* qrow = q + size_t(bh) * D;
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
    const float ah = 0.5f * af;
    float4* f = reinterpret_cast<float4*>(&L.fin[lane >> 4][8 * (lane & 15)]);
    f[0] = make_float4(fs.acc[0] * ah, fs.acc[1] * ah, fs.acc[2] * ah, fs.acc[3] * ah);
    f[1] = make_float4(fs.acc[4] * ah, fs.acc[5] * ah, fs.acc[6] * ah, fs.acc[7] * ah);
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[k] += L.fin[lane & 3][16 * k + (lane >> 2)];
    wave_lds_sync();
  };
  int n = 0;
  for (int u = sp.p0 + wave; u < p1; u += kWaves, ++n) {
    prio_by_work_left((p1 - u + kWaves - 1) / kWaves);
    PageRegs<G> pr;
    load_page<G>(pr, pages + size_t(u) * PB, lane);
    compute_page<G>(pr, page_nvalid(a.G, a.P, u), qs0, qs1, L.qp, L.ph, st, lane);
    if ((n & 3) == wave && chunk < t1) next_chunk();
  }
  while (chunk < t1) next_chunk();

  // this wave's state -> LDS in channel order (accumulator back to full units)
  const float l_tot = wave_sum(st.l);
  const float v_tot = wave_sum(st.vmin);
#pragma unroll
  for (int k = 0; k < 8; ++k) st.acc[k] = quad_sum(st.acc[k]);
  if ((lane & 3) == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) L.fin[0][16 * k + (lane >> 2)] = fmaf(2.0f, st.acc[k], v_tot);
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
