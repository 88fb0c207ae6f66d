// HIP kernels of the OTT path for gfx950 (CDNA4, wave64).
//
// Method: "Accurate KV Cache Quantization with Outlier Tokens Tracing"
// (arXiv 2505.10938); [Blog] = zijie-tian.site summary page, [Abs] =
// sciencestack.ai page (abstract and figure captions).
//
//   append_kernel    fp16 window update ([Blog] 3.3, residual window)
//   quantize_kernel  quantization stage: Key norms, pool competition, 2-bit
//                    pages ([Blog] 3.1, 3.2, flowchart; [Abs] Fig. 2 bottom)
//   decode_kernel    decoding stage over the three caches with one online
//                    softmax ([Blog] 3.3 and flowchart; [Abs] Fig. 2 top)
//   combine_kernel   merge of split-K partial softmax states
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ott_kernels.h"

namespace ott {
namespace {

constexpr int D = kHeadDim;
constexpr int kRingFlag = 0x40000000;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Arena addressing
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t* counters(const Arena& a, int bh) {
  return reinterpret_cast<int32_t*>(a.base + a.off_counters) + size_t(bh) * 4;
}
__device__ __forceinline__ uint8_t* page_ptr(const Arena& a, int bh, int n) {
  return a.base + a.off_pages + (size_t(bh) * a.nb_max + n) * a.page_bytes;
}
__device__ __forceinline__ __half* pool_k(const Arena& a, int buf, int bh) {
  return reinterpret_cast<__half*>(a.base + a.off_pool_k) +
         ((size_t(buf) * a.B * a.Hkv + bh) * a.P) * D;
}
__device__ __forceinline__ __half* pool_v(const Arena& a, int buf, int bh) {
  return reinterpret_cast<__half*>(a.base + a.off_pool_v) +
         ((size_t(buf) * a.B * a.Hkv + bh) * a.P) * D;
}
__device__ __forceinline__ int32_t* pool_pos(const Arena& a, int buf, int bh) {
  return reinterpret_cast<int32_t*>(a.base + a.off_pool_pos) +
         (size_t(buf) * a.B * a.Hkv + bh) * a.P;
}
__device__ __forceinline__ double* pool_n2(const Arena& a, int buf, int bh) {
  return reinterpret_cast<double*>(a.base + a.off_pool_n2) +
         (size_t(buf) * a.B * a.Hkv + bh) * a.P;
}
__device__ __forceinline__ __half* ring_k(const Arena& a, int bh) {
  return reinterpret_cast<__half*>(a.base + a.off_ring_k) + size_t(bh) * a.C * D;
}
__device__ __forceinline__ __half* ring_v(const Arena& a, int bh) {
  return reinterpret_cast<__half*>(a.base + a.off_ring_v) + size_t(bh) * a.C * D;
}

// Page geometry (byte offsets inside one page).
__host__ __device__ constexpr int kcode_off(int) { return 0; }
__host__ __device__ constexpr int vcode_off(int G) { return G * D / 4; }
__host__ __device__ constexpr int kmeta_off(int G) { return G * D / 4 + D * G / 4; }
__host__ __device__ constexpr int vmeta_off(int G) { return kmeta_off(G) + 4 * D; }

// Members of page n: a page holds the group plus the pool minus the new pool
// (the pool holds min(P, G*n) tokens before the n-th quantize step).
__device__ __forceinline__ int page_nvalid(int G, int P, int n) {
  const int pc = min(P, G * n);
  return G + pc - min(P, pc + G);
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(Arena a, const uint4* __restrict__ k,
                                                     const uint4* __restrict__ v,
                                                     AppendCounts cnt) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int bh = b * a.Hkv + h;
  const int n = cnt.uniform >= 0 ? cnt.uniform : int(cnt.n[b]);
  if (n == 0) return;
  int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2];
  uint4* rk = reinterpret_cast<uint4*>(ring_k(a, bh));
  uint4* rv = reinterpret_cast<uint4*>(ring_v(a, bh));
  const size_t src = size_t(bh) * cnt.max_new * (D / 8);
  for (int i = threadIdx.x; i < n * (D / 8); i += blockDim.x) {
    const int t = i / (D / 8), c = i % (D / 8);
    const int slot = (head + r_cnt + t) % a.C;
    rk[size_t(slot) * (D / 8) + c] = k[src + i];
    rv[size_t(slot) * (D / 8) + c] = v[src + i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ctr[0] += n;
    ctr[1] = r_cnt + n;
  }
}

// ---------------------------------------------------------------------------
// quantize: one work-group per (sequence, KV head) with a full window
// ---------------------------------------------------------------------------

// 2-bit code of x against (min m, scale s): clamp(rint((x - m) / s), 0, 3).
// x - m and the division are single IEEE fp32 operations (correctly rounded);
// rintf rounds half to even.
__device__ __forceinline__ uint32_t qcode(float x, float m, float s) {
  if (s == 0.0f) return 0u;
  const float y = __fdiv_rn(__fsub_rn(x, m), s);
  const float r = fminf(fmaxf(rintf(y), 0.0f), 3.0f);
  return uint32_t(r);
}

struct QuantLds {
  double* n2;
  int* pos;
  int* src;
  int* rank;
  int* mem;
  float* kmin;
  float* kscale;
  float* vmin;
  float* vscale;
};

__device__ __forceinline__ QuantLds quant_lds(uint8_t* base, int NCmax, int G) {
  QuantLds q;
  q.n2 = reinterpret_cast<double*>(base);
  q.pos = reinterpret_cast<int*>(q.n2 + NCmax);
  q.src = q.pos + NCmax;
  q.rank = q.src + NCmax;
  q.mem = q.rank + NCmax;
  q.kmin = reinterpret_cast<float*>(q.mem + G);
  q.kscale = q.kmin + D;
  q.vmin = q.kscale + D;
  q.vscale = q.vmin + G;
  return q;
}

__global__ __launch_bounds__(256) void quantize_kernel(Arena a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const int h = blockIdx.x, b = blockIdx.y;
  const int bh = b * a.Hkv + h;
  const int G = a.G, P = a.P, C = a.C;
  int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  if (r_cnt < C) return;  // window not full: nothing to do for this sequence
  const int tid = threadIdx.x;
  const int pc = min(P, G * nb);  // pool tokens before this step
  const int NC = pc + G;          // candidates: pool + group
  const int npc = min(P, NC);     // pool tokens after this step
  const int n_valid = NC - npc;   // page members
  const int cur = nb & 1, nxt = cur ^ 1;
  QuantLds s = quant_lds(lds_raw, P + G, G);

  const __half* pk = pool_k(a, cur, bh);
  const __half* pv = pool_v(a, cur, bh);
  const __half* rk = ring_k(a, bh);
  const __half* rv = ring_v(a, bh);
  auto krow = [&](int src) -> const __half* {
    return (src & kRingFlag) ? rk + size_t(src & ~kRingFlag) * D : pk + size_t(src) * D;
  };
  auto vrow = [&](int src) -> const __half* {
    return (src & kRingFlag) ? rv + size_t(src & ~kRingFlag) * D : pv + size_t(src) * D;
  };

  // 1. candidates; squared Key norms of the group, fp64 in channel order
  for (int i = tid; i < NC; i += blockDim.x) {
    if (i < pc) {
      s.n2[i] = pool_n2(a, cur, bh)[i];
      s.pos[i] = pool_pos(a, cur, bh)[i];
      s.src[i] = i;
    } else {
      const int j = i - pc;
      const int slot = (head + j) % C;
      const uint4* row = reinterpret_cast<const uint4*>(rk + size_t(slot) * D);
      double acc = 0.0;
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 w = row[c8];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double lo = double(__half2float(__ushort_as_half(uint16_t(ws[e] & 0xffffu))));
          const double hi = double(__half2float(__ushort_as_half(uint16_t(ws[e] >> 16))));
          acc = acc + lo * lo;
          acc = acc + hi * hi;
        }
      }
      s.n2[i] = acc;
      s.pos[i] = G * nb + j;
      s.src[i] = slot | kRingFlag;
    }
  }
  __syncthreads();

  // 2. rank under (norm, position)
  for (int i = tid; i < NC; i += blockDim.x) {
    const double ni = s.n2[i];
    const int pi = s.pos[i];
    int r = 0;
    for (int j = 0; j < NC; ++j) {
      const double nj = s.n2[j];
      r += (nj < ni) || (nj == ni && s.pos[j] < pi);
    }
    s.rank[i] = r;
  }
  __syncthreads();

  // 3. members (rank >= npc) in position order
  for (int i = tid; i < NC; i += blockDim.x) {
    if (s.rank[i] >= npc) {
      const int pi = s.pos[i];
      int idx = 0;
      for (int j = 0; j < NC; ++j) idx += (s.rank[j] >= npc) && (s.pos[j] < pi);
      s.mem[idx] = i;
    }
  }
  __syncthreads();

  uint8_t* pg = page_ptr(a, bh, nb);
  // 4. Key (min, scale) per channel over the members
  if (tid < D) {
    float lo = 0.f, hi = 0.f;
    if (n_valid > 0) {
      lo = INFINITY;
      hi = -INFINITY;
      for (int t = 0; t < n_valid; ++t) {
        const float x = __half2float(krow(s.src[s.mem[t]])[tid]);
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
    }
    const __half sc = __float2half_rn(__fdiv_rn(__fsub_rn(hi, lo), 3.0f));
    s.kmin[tid] = lo;
    s.kscale[tid] = __half2float(sc);
    const uint32_t word =
        uint32_t(__half_as_ushort(__float2half_rn(lo))) | (uint32_t(__half_as_ushort(sc)) << 16);
    reinterpret_cast<uint32_t*>(pg + kmeta_off(G))[tid] = word;
  }
  // 5. Value (min, scale) per member token over its channels
  for (int t = tid; t < G; t += blockDim.x) {
    uint32_t word = 0;
    float lo = 0.f, scf = 0.f;
    if (t < n_valid) {
      const uint4* row = reinterpret_cast<const uint4*>(vrow(s.src[s.mem[t]]));
      float mn = INFINITY, mx = -INFINITY;
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 w = row[c8];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __half2float(__ushort_as_half(uint16_t(ws[e] & 0xffffu)));
          const float x1 = __half2float(__ushort_as_half(uint16_t(ws[e] >> 16)));
          mn = fminf(mn, fminf(x0, x1));
          mx = fmaxf(mx, fmaxf(x0, x1));
        }
      }
      const __half sc = __float2half_rn(__fdiv_rn(__fsub_rn(mx, mn), 3.0f));
      lo = mn;
      scf = __half2float(sc);
      word = uint32_t(__half_as_ushort(__float2half_rn(mn))) |
             (uint32_t(__half_as_ushort(sc)) << 16);
    }
    s.vmin[t] = lo;
    s.vscale[t] = scf;
    reinterpret_cast<uint32_t*>(pg + vmeta_off(G))[t] = word;
  }
  __syncthreads();

  // 6. K codes, token-major: dword (t, j) = channels 16j..16j+15 of member t
  uint32_t* kc = reinterpret_cast<uint32_t*>(pg + kcode_off(G));
  for (int w = tid; w < G * (D / 16); w += blockDim.x) {
    const int t = w / (D / 16), j = w % (D / 16);
    uint32_t word = 0;
    if (t < n_valid) {
      const __half* row = krow(s.src[s.mem[t]]) + 16 * j;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const int c = 16 * j + cc;
        word |= qcode(__half2float(row[cc]), s.kmin[c], s.kscale[c]) << (2 * cc);
      }
    }
    kc[w] = word;
  }
  // 7. V codes, channel-major: dword (c, j) = slots 16j..16j+15 of channel c
  uint32_t* vc = reinterpret_cast<uint32_t*>(pg + vcode_off(G));
  const int vdw = G / 16;
  for (int w = tid; w < D * vdw; w += blockDim.x) {
    const int c = w / vdw, j = w % vdw;
    uint32_t word = 0;
#pragma unroll 4
    for (int cc = 0; cc < 16; ++cc) {
      const int t = 16 * j + cc;
      if (t < n_valid)
        word |= qcode(__half2float(vrow(s.src[s.mem[t]])[c]), s.vmin[t], s.vscale[t]) << (2 * cc);
    }
    vc[w] = word;
  }
  // 8. the new pool, slot = rank, into the other buffer
  __half* nk = pool_k(a, nxt, bh);
  __half* nv = pool_v(a, nxt, bh);
  for (int w = tid; w < NC * (D / 8); w += blockDim.x) {
    const int i = w / (D / 8), c8 = w % (D / 8);
    const int r = s.rank[i];
    if (r < npc) {
      reinterpret_cast<uint4*>(nk + size_t(r) * D)[c8] =
          reinterpret_cast<const uint4*>(krow(s.src[i]))[c8];
      reinterpret_cast<uint4*>(nv + size_t(r) * D)[c8] =
          reinterpret_cast<const uint4*>(vrow(s.src[i]))[c8];
      if (c8 == 0) {
        pool_pos(a, nxt, bh)[r] = s.pos[i];
        pool_n2(a, nxt, bh)[r] = s.n2[i];
      }
    }
  }
  // 9. member positions (tests only)
  int32_t* ppos = reinterpret_cast<int32_t*>(a.base + a.off_page_pos) +
                  (size_t(bh) * a.nb_max + nb) * G;
  for (int t = tid; t < G; t += blockDim.x) ppos[t] = t < n_valid ? s.pos[s.mem[t]] : -1;
  if (tid == 0)
    reinterpret_cast<int32_t*>(a.base + a.off_page_nvalid)[size_t(bh) * a.nb_max + nb] = n_valid;
  __syncthreads();
  if (tid == 0) {
    ctr[1] = r_cnt - G;
    ctr[2] = (head + G) % C;
    ctr[3] = nb + 1;
  }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 1, 64); }

// Orders this wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float lo_f(uint32_t w) {
  return __half2float(__ushort_as_half(uint16_t(w & 0xffffu)));
}
__device__ __forceinline__ float hi_f(uint32_t w) {
  return __half2float(__ushort_as_half(uint16_t(w >> 16)));
}

// Online softmax state of one wave for one query head (scores in log2 units).
struct WaveState {
  float m;        // running max (wave-uniform)
  float l;        // partial sum of weights (this lane's tokens)
  float vmin;     // partial sum of p_t * min_t over quantized tokens
  float accq[4];  // quantized-V accumulator: channel 32k + lane/2, token half lane&1
  float accf[2];  // fp16-V accumulator: channels 2*lane, 2*lane+1
};

// Dot of 16 2-bit codes (one dword, code i in bits 2i..2i+1) with 16 weights.
// The FP4 (E2M1) view of a nibble whose two high bits are zero is code/2, so
// two mask operations turn the dword into 8 + 8 FP4 values and each byte
// converts to two floats in one instruction. Weights must be pre-doubled.
__device__ __forceinline__ float dot16_codes(uint32_t w, const float4& c0, const float4& c1,
                                             const float4& c2, const float4& c3, float acc) {
  const uint32_t ev = w & 0x33333333u;         // codes 0,2 of every byte
  const uint32_t od = (w >> 2) & 0x33333333u;  // codes 1,3 of every byte
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

__device__ __forceinline__ uint32_t dw(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// One quantized page for one query head.
//   K side: lane pair (2i, 2i+1) owns token 32k+i of pass k; each lane takes 64
//   channels. V side: lane pair owns channel 32k+i; each lane takes half of the
//   page's slots.
template <int G>
__device__ __forceinline__ void decode_page(const uint8_t* __restrict__ pg, int n_valid, float qs0,
                                            float qs1, float* qp, float* ps, WaveState& st,
                                            int lane) {
  constexpr int KP = G / 32;   // K passes of 32 tokens
  constexpr int VQ = G / 128;  // uint4 per V channel half (G/8 bytes); G=64 uses one uint2
  const int hh = lane & 1, tl = lane >> 1;

  uint4 kc[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k)
    kc[k] = *reinterpret_cast<const uint4*>(pg + (32 * k + tl) * (D / 4) + 16 * hh);
  uint32_t vcw[4][VQ > 0 ? VQ * 4 : 2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint8_t* src = pg + vcode_off(G) + (32 * k + tl) * (G / 4) + hh * (G / 8);
    if constexpr (VQ > 0) {
#pragma unroll
      for (int q = 0; q < VQ; ++q) {
        const uint4 t = reinterpret_cast<const uint4*>(src)[q];
        vcw[k][4 * q + 0] = t.x;
        vcw[k][4 * q + 1] = t.y;
        vcw[k][4 * q + 2] = t.z;
        vcw[k][4 * q + 3] = t.w;
      }
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      vcw[k][0] = t.x;
      vcw[k][1] = t.y;
    }
  }
  uint32_t vm[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k)
    vm[k] = reinterpret_cast<const uint32_t*>(pg + vmeta_off(G))[32 * k + tl];
  const uint2 km = reinterpret_cast<const uint2*>(pg + kmeta_off(G))[lane];

  // q' = q * scale per channel (doubled for the FP4 code/2 view); bias = q . min
  const float qa = 2.0f * qs0 * hi_f(km.x), qb = 2.0f * qs1 * hi_f(km.y);
  float bias = qs0 * lo_f(km.x) + qs1 * lo_f(km.y);
  *reinterpret_cast<float2*>(qp + 2 * lane) = make_float2(qa, qb);
  bias = wave_sum(bias);
  wave_lds_sync();

  float z[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) z[k] = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4* qv = reinterpret_cast<const float4*>(qp + 64 * hh + 16 * j);
    const float4 c0 = qv[0], c1 = qv[1], c2 = qv[2], c3 = qv[3];
#pragma unroll
    for (int k = 0; k < KP; ++k) z[k] = dot16_codes(dw(kc[k], j), c0, c1, c2, c3, z[k]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    z[k] = pair_sum(z[k]) + bias;
    if (32 * k + tl >= n_valid) z[k] = -INFINITY;
    mx = fmaxf(mx, z[k]);
  }
  mx = wave_max(mx);
  if (mx == -INFINITY) return;
  const float m_new = fmaxf(st.m, mx);
  const float alpha = (st.m == -INFINITY) ? 0.f : exp2f(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  st.vmin *= alpha;
#pragma unroll
  for (int k = 0; k < 4; ++k) st.accq[k] *= alpha;
  st.accf[0] *= alpha;
  st.accf[1] *= alpha;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const float p = exp2f(z[k] - m_new);
    if (hh == 0) {
      st.l += p;
      st.vmin = fmaf(p, lo_f(vm[k]), st.vmin);
      ps[32 * k + tl] = 2.0f * p * hi_f(vm[k]);
    }
  }
  wave_lds_sync();
  constexpr int VDW = G / 32;  // dwords per channel half
#pragma unroll
  for (int j = 0; j < VDW; ++j) {
    const float4* pv = reinterpret_cast<const float4*>(ps + hh * (G / 2) + 16 * j);
    const float4 c0 = pv[0], c1 = pv[1], c2 = pv[2], c3 = pv[3];
#pragma unroll
    for (int k = 0; k < 4; ++k) st.accq[k] = dot16_codes(vcw[k][j], c0, c1, c2, c3, st.accq[k]);
  }
  wave_lds_sync();
}

// Up to 64 fp16 tokens (pool first, then the window) for one query head.
// Lane i scores token base+i; then every lane accumulates its two channels.
__device__ __forceinline__ void decode_fp16_chunk(const __half* pk, const __half* pv,
                                                  const __half* rk, const __half* rv, int pc,
                                                  int n16, int head, int C, int base,
                                                  const uint32_t* qh, float qscale, float* ps,
                                                  WaveState& st, int lane) {
  const int cnt = min(64, n16 - base);
  const int i = base + lane;
  float z = -INFINITY;
  if (lane < cnt) {
    const __half* row = i < pc ? pk + size_t(i) * D : rk + size_t((head + i - pc) % C) * D;
    const uint4* r4 = reinterpret_cast<const uint4*>(row);
    const uint4* q4 = reinterpret_cast<const uint4*>(qh);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 kv = r4[c], qv = q4[c];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kv.x), __builtin_bit_cast(f16x2, qv.x), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kv.y), __builtin_bit_cast(f16x2, qv.y), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kv.z), __builtin_bit_cast(f16x2, qv.z), acc, false);
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kv.w), __builtin_bit_cast(f16x2, qv.w), acc, false);
    }
    z = acc * qscale;
  }
  const float mx = wave_max(z);
  const float m_new = fmaxf(st.m, mx);
  const float alpha = (st.m == -INFINITY) ? 0.f : exp2f(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  st.vmin *= alpha;
#pragma unroll
  for (int k = 0; k < 4; ++k) st.accq[k] *= alpha;
  st.accf[0] *= alpha;
  st.accf[1] *= alpha;
  const float p = exp2f(z - m_new);
  st.l += p;
  ps[lane] = p;
  wave_lds_sync();
  float a0 = 0.f, a1 = 0.f;
  for (int t = 0; t < cnt; ++t) {
    const int j = base + t;
    const __half* row = j < pc ? pv + size_t(j) * D : rv + size_t((head + j - pc) % C) * D;
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
    const float pt = ps[t];
    a0 = fmaf(pt, lo_f(w), a0);
    a1 = fmaf(pt, hi_f(w), a1);
  }
  st.accf[0] += a0;
  st.accf[1] += a1;
  wave_lds_sync();
}

template <int G>
__global__ __launch_bounds__(256) void decode_kernel(Arena a, const __half* __restrict__ q,
                                                     __half* __restrict__ out, int S) {
  __shared__ __align__(16) float qp_s[4][D];
  __shared__ __align__(16) float ps_s[4][G > 64 ? G : 64];
  __shared__ __align__(16) uint32_t qh_s[4][D / 2];
  __shared__ __align__(16) float mg_acc[4][D];
  __shared__ float mg_m[4], mg_l[4];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int NQ = a.Hq / a.Hkv;
  const int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  const int pc = min(a.P, a.G * nb);
  const int n16 = pc + r_cnt;
  const int U = nb + (n16 + kFp16Chunk - 1) / kFp16Chunk;
  const int u0 = int(int64_t(s) * U / S), u1 = int(int64_t(s + 1) * U / S);
  const int wph = NQ >= 4 ? 1 : 4 / NQ;  // waves per query head
  const int hpr = 4 / wph;               // query heads per round
  const int rounds = (NQ + hpr - 1) / hpr;
  const float qscale = a.sm_scale * kLog2e;
  const int buf = nb & 1;
  const __half* pk = pool_k(a, buf, bh);
  const __half* pv = pool_v(a, buf, bh);
  const __half* rk = ring_k(a, bh);
  const __half* rv = ring_v(a, bh);

  for (int r = 0; r < rounds; ++r) {
    const int qi = r * hpr + wave / wph;
    const int stripe = wave % wph;
    if (qi < NQ) {
      const int qh = h * NQ + qi;
      const uint32_t q2 = reinterpret_cast<const uint32_t*>(q + (size_t(b) * a.Hq + qh) * D)[lane];
      qh_s[wave][lane] = q2;
      const float qs0 = lo_f(q2) * qscale, qs1 = hi_f(q2) * qscale;
      wave_lds_sync();
      WaveState st;
      st.m = -INFINITY;
      st.l = 0.f;
      st.vmin = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) st.accq[k] = 0.f;
      st.accf[0] = st.accf[1] = 0.f;
      for (int u = u0 + stripe; u < u1; u += wph) {
        if (u < nb) {
          decode_page<G>(page_ptr(a, bh, u), page_nvalid(a.G, a.P, u), qs0, qs1, qp_s[wave],
                         ps_s[wave], st, lane);
        } else {
          decode_fp16_chunk(pk, pv, rk, rv, pc, n16, head, a.C, (u - nb) * kFp16Chunk,
                            qh_s[wave], qscale, ps_s[wave], st, lane);
        }
      }
      // this wave's state -> LDS, in plain channel order
      const float lt = wave_sum(st.l);
      const float vt = wave_sum(st.vmin);
#pragma unroll
      for (int k = 0; k < 4; ++k) st.accq[k] = pair_sum(st.accq[k]);
      if ((lane & 1) == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) mg_acc[wave][32 * k + (lane >> 1)] = st.accq[k];
      }
      wave_lds_sync();
      float2 c2 = *reinterpret_cast<float2*>(&mg_acc[wave][2 * lane]);
      c2.x += st.accf[0] + vt;
      c2.y += st.accf[1] + vt;
      *reinterpret_cast<float2*>(&mg_acc[wave][2 * lane]) = c2;
      if (lane == 0) {
        mg_m[wave] = st.m;
        mg_l[wave] = lt;
      }
    }
    __syncthreads();
    // merge the waves of each query head of this round
    for (int j = threadIdx.x; j < hpr * D; j += blockDim.x) {
      const int hr = j / D, c = j % D;
      const int qi2 = r * hpr + hr;
      if (qi2 >= NQ) continue;
      float M = -INFINITY;
      for (int w = hr * wph; w < (hr + 1) * wph; ++w) M = fmaxf(M, mg_m[w]);
      float Ls = 0.f, A = 0.f;
      for (int w = hr * wph; w < (hr + 1) * wph; ++w) {
        const float f = (mg_m[w] == -INFINITY) ? 0.f : exp2f(mg_m[w] - M);
        Ls = fmaf(mg_l[w], f, Ls);
        A = fmaf(mg_acc[w][c], f, A);
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

// Merge of S split-K partial states per (sequence, query head).
__global__ __launch_bounds__(128) void combine_kernel(Arena a, __half* __restrict__ out, int S) {
  const int bq = blockIdx.x;  // b * Hq + qh
  const int c = threadIdx.x;
  const float* part = reinterpret_cast<const float*>(a.base + a.off_partials) +
                      size_t(bq) * a.max_splits * (2 + D);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[s * (2 + D)]);
  float Ls = 0.f, A = 0.f;
  for (int s = 0; s < S; ++s) {
    const float m = part[s * (2 + D)];
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    Ls = fmaf(part[s * (2 + D) + 1], f, Ls);
    A = fmaf(part[s * (2 + D) + 2 + c], f, A);
  }
  out[size_t(bq) * D + c] = __float2half_rn(A / Ls);
}

}  // namespace

hipError_t launch_append(const Arena& a, const void* k, const void* v, const AppendCounts& n,
                         hipStream_t s) {
  dim3 grid(a.Hkv, a.B);
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, s, a, static_cast<const uint4*>(k),
                     static_cast<const uint4*>(v), n);
  return hipGetLastError();
}

size_t quantize_lds_bytes(int G, int P) {
  const size_t nc = size_t(P) + G;
  return nc * sizeof(double) + 3 * nc * sizeof(int) + G * sizeof(int) + 2 * D * sizeof(float) +
         2 * size_t(G) * sizeof(float);
}

hipError_t launch_quantize(const Arena& a, hipStream_t s) {
  dim3 grid(a.Hkv, a.B);
  hipLaunchKernelGGL(quantize_kernel, grid, dim3(256), quantize_lds_bytes(a.G, a.P), s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Arena& a, const void* q, void* out, int S, hipStream_t s) {
  const dim3 grid(unsigned(a.B) * a.Hkv * S);
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  switch (a.G) {
    case 64: hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(256), 0, s, a, qh, oh, S); break;
    case 128: hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(256), 0, s, a, qh, oh, S); break;
    case 256: hipLaunchKernelGGL(decode_kernel<256>, grid, dim3(256), 0, s, a, qh, oh, S); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(a.B) * a.Hq), dim3(D), 0, s, a, oh, S);
  return hipGetLastError();
}

}  // namespace ott
