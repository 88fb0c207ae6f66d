// Decoding stage for grouped query heads (several query heads per KV head) on
// gfx950 matrix cores.
//
// Same computation as the one-head kernel ([Blog] zijie-tian.site summary,
// section 3.3 flowchart; [Abs] sciencestack.ai, Figure 2 top): scores of the
// quantized Keys, the window Keys and the pool Keys go under one softmax and
// the weights multiply the matching Values. With QB query heads sharing a
// page, both products over the page are small dense contractions:
//
//   scores  z[h][t] = bias[h] + sum_c q'[h][c] * kcode[t][c]   (QB x 128 x G)
//   values  o[h][c] += sum_t p'[h][t] * vcode[c][t]            (QB x G x 128)
//
// with q'[h][c] = qs[h][c] * scale_c and p'[h][t] = p[h][t] * scale_t. Both
// run on v_mfma_f32_16x16x32_f16. A 2-bit code whose two high neighbour bits
// are masked off is the FP4 (E2M1) value code/2, which one conversion per two
// codes turns into fp16 (0, 0.5, 1, 1.5: exact and normal); the factor 2
// returns after the products. q' enters as an fp16 pair hi + lo (22
// significant bits), p' as one fp16 value.
#include "ott_decode_common.h"

namespace ott {
namespace {
using namespace dev;
using namespace dec;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// D(16x16) += A(16x32) B(32x16). Lane l holds A row l%16, B column l%16, the
// k-slots 8(l/16)..8(l/16)+7 of both, and D rows 4(l/16)..4(l/16)+3 of column
// l%16.
__device__ __forceinline__ f4 mfma16(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One dword of 16 codes (code n in bits 2n..2n+1) as the B operands of two
// MFMA steps, as code/2: slot e of step h holds code 8h + kPerm[e] (each FP4
// conversion yields codes 0 and 2, or 1 and 3, of one byte).
__device__ __forceinline__ void codes_b(uint32_t w, h8& b0, h8& b1) {
  const uint32_t ev = w & 0x33333333u;         // codes 0 and 2 of every byte
  const uint32_t od = (w >> 2) & 0x33333333u;  // codes 1 and 3 of every byte
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 0);
  const h2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 0);
  const h2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 1);
  const h2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 1);
  const h2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 2);
  const h2 o2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 2);
  const h2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 3);
  const h2 o3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 3);
  b0 = h8{e0[0], e0[1], o0[0], o0[1], e1[0], e1[1], o1[0], o1[1]};
  b1 = h8{e2[0], e2[1], o2[0], o2[1], e3[0], e3[1], o3[0], o3[1]};
}

// Code (channel or token) offset of slot e inside an MFMA step.
__host__ __device__ constexpr int kPerm(int e) { return (e & ~3) | ((e & 1) << 1) | ((e >> 1) & 1); }

// Shapes for page size G and QB query heads per pass.
//   K: tile T = tokens 16T..16T+15 (B column = token); lane group g covers
//      channels 32g..32g+31 of the token's code row, step cb the channels
//      32g + 8cb + kPerm(slot).
//   V: tile ct = channels 16ct..16ct+15 (B column = channel); lane group g
//      covers tokens g*G/4..g*G/4+G/4-1 of the channel's code row, step kb the
//      tokens g*G/4 + 8kb + kPerm(slot).
//   A rows: query head h at row h (its q' hi part and p'), q' lo part at row
//      QB + h; with QB = 16 the lo parts fill a second 16-row array.
template <int G, int QB>
struct Geo {
  static constexpr int NA = QB <= 8 ? 1 : 2;       // 16-row arrays of q'
  static constexpr int ZR = QB <= 8 ? 2 * QB : QB;  // score values kept per token
  static constexpr int KT = G / 16;                 // K tiles
  static constexpr int VDW = G / 64;                // V code dwords per lane and channel
  static constexpr int KB = G / 32;                 // V steps
  static constexpr int NP = G / 2;                  // token pairs (t, t + 2)
  static constexpr int PPL = (NP + 63) / 64;        // pairs per lane
  static constexpr int QPL = (QB + 3) / 4;          // query heads per lane in the q' step
  static constexpr int ZS0 = G * ZR > 4 * D ? G * ZR : 4 * D;
  static constexpr int ZS = ZS0 > QB * D ? ZS0 : QB * D;  // floats
  // A operands live in blocks of 16 rows x 16 bytes, padded to 272 bytes so
  // that writes of one row across blocks spread over the LDS banks
  static constexpr int kBlk = 272;
  static constexpr int NBLK = NA * 16 > KB * 4 ? NA * 16 : KB * 4;
};

// First token of pair pi; the pair is (t, t + 2) and fills the dword p (slots
// 2p, 2p + 1) of A row h in V step kb for lane group g.
template <int G>
__device__ __forceinline__ int pair_token(int pi) {
  const int g = pi / (G / 8), rem = pi % (G / 8), kb = rem >> 2, p = rem & 3;
  return g * (G / 4) + 8 * kb + (p & 1) + 4 * (p >> 1);
}

template <int G, int QB>
struct alignas(16) GqaLds {
  // q' A operands: block (a * 4 + cb) * 4 + lane group; p' A operands: block kb * 4 + lane group
  uint8_t ab[Geo<G, QB>::NBLK * Geo<G, QB>::kBlk];
  float zs[Geo<G, QB>::ZS];  // page scores [token][row]; fp16 fold; final state
  float bias[16];
  __device__ __forceinline__ h8* row(int blk, int r) {
    return reinterpret_cast<h8*>(ab + blk * Geo<G, QB>::kBlk + 16 * r);
  }
};

template <int QB>
struct GqaState {
  float m[QB];     // running max per query head (wave-uniform)
  float l[QB];     // this lane's share of the running sums
  float vmin[QB];  // this lane's share of sum p_t * min_t
  f4 acc[8];       // sum p'_t c_t / 2: rows 4(lane>>4)+r, channel 16ct + (lane&15)
};

// Per-lane value of a per-head array for D row 4g + r.
template <int QB>
__device__ __forceinline__ float row_pick(const float (&v)[QB], int g, int r) {
  float x = v[r % QB];
#pragma unroll
  for (int gg = 1; gg < (QB + 3) / 4; ++gg)
    if (g % ((QB + 3) / 4) == gg) x = v[4 * gg + r];
  return x;
}

// Wave-wide maxima of N values per lane, the N reductions in lockstep.
template <int N>
__device__ __forceinline__ void wave_max_n(float (&x)[N]) {
#pragma unroll
  for (int h = 0; h < N; ++h) x[h] = fmaxf(x[h], dpp<kQuadSwap1>(x[h]));
#pragma unroll
  for (int h = 0; h < N; ++h) x[h] = fmaxf(x[h], dpp<kQuadSwap2>(x[h]));
#pragma unroll
  for (int h = 0; h < N; ++h) x[h] = fmaxf(x[h], dpp<kHalfMirror>(x[h]));
#pragma unroll
  for (int h = 0; h < N; ++h) x[h] = fmaxf(x[h], dpp<kRowMirror>(x[h]));
#pragma unroll
  for (int h = 0; h < N; ++h) {
    const f32x2 p = swap16(x[h]);
    x[h] = fmaxf(p.x, p.y);
  }
#pragma unroll
  for (int h = 0; h < N; ++h) {
    const f32x2 p = swap32(x[h]);
    x[h] = fmaxf(p.x, p.y);
  }
}

// The part of a page one lane reads from memory.
template <int G>
struct GqaPage {
  static constexpr int KT = G / 16, VDW = G / 64, PPL = (G / 2 + 63) / 64;
  uint4 kmA, kmB;        // K (min, scale) of the lane's q' channels 8j..8j+7
  uint2 kc[KT];          // K codes: tile T, token 16T + (lane&15), lane group's 32 channels
  uint32_t vm[PPL][2];   // V (min, scale) of the lane's token pairs
  uint32_t vc[8][VDW];   // V codes: tile ct, channel 16ct + (lane&15), lane group's tokens
};

template <int G>
__device__ __forceinline__ void gqa_load(GqaPage<G>& r, const uint8_t* __restrict__ pg, int lane) {
  constexpr int NP = G / 2;
  const int j = lane & 15, g = lane >> 4;
  const int c0 = 8 * j;  // q' chunk of this lane: channels c0..c0+7 (lane group j>>2, step j&3)
  r.kmA = ld_nt4(pg + kmeta_off(G) + 4 * c0);
  r.kmB = ld_nt4(pg + kmeta_off(G) + 4 * (c0 + 4));
#pragma unroll
  for (int T = 0; T < GqaPage<G>::KT; ++T) r.kc[T] = ld_nt2(pg + (16 * T + j) * (D / 4) + 8 * g);
#pragma unroll
  for (int k = 0; k < GqaPage<G>::PPL; ++k) {
    const int t0 = pair_token<G>(min(lane + 64 * k, NP - 1));
    r.vm[k][0] = ld_nt1(pg + vmeta_off(G) + 4 * t0);
    r.vm[k][1] = ld_nt1(pg + vmeta_off(G) + 4 * (t0 + 2));
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const uint8_t* src = pg + vcode_off(G) + (16 * ct + j) * (G / 4) + g * (G / 16);
    if constexpr (GqaPage<G>::VDW == 4) {
      const uint4 t = ld_nt4(src);
      r.vc[ct][0] = t.x; r.vc[ct][1] = t.y; r.vc[ct][2] = t.z; r.vc[ct][3] = t.w;
    } else if constexpr (GqaPage<G>::VDW == 2) {
      const uint2 t = ld_nt2(src);
      r.vc[ct][0] = t.x; r.vc[ct][1] = t.y;
    } else {
      r.vc[ct][0] = ld_nt1(src);
    }
  }
}

template <int G, int QB>
__device__ __forceinline__ void gqa_page(const GqaPage<G>& r, int n_valid,
                                         const float (&qs)[Geo<G, QB>::QPL][8],
                                         GqaLds<G, QB>& L, GqaState<QB>& st, int lane) {
  using Gm = Geo<G, QB>;
  const int j = lane & 15, g = lane >> 4;
  const int cg = j >> 2, cb = j & 3;
  const uint4 &kmA = r.kmA, &kmB = r.kmB;
  const auto& kc = r.kc;
  const auto& vm = r.vm;
  const auto& vc = r.vc;

  // ---- q' = qs * scale_c for the lane's 8 channels (slot order); with codes
  // entering as c/2: z = sum qs min_c + 2 sum q' c/2
  float scl[8], mnv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = kPerm(e);
    const uint32_t w = c < 4 ? dw(kmA, c) : dw(kmB, c - 4);
    mnv[e] = lo_f(w);
    scl[e] = hi_f(w);
  }
  float qp[Gm::QPL][8], bp[Gm::QPL];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < Gm::QPL; ++k) {
    bp[k] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qp[k][e] = qs[k][e] * scl[e];
      bp[k] = fmaf(qs[k][e], mnv[e], bp[k]);
      amax = fmaxf(amax, fabsf(qp[k][e]));
    }
  }
  // keep |q'| below 2^15 in fp16: scale by a power of two if the page needs it
  const float mx = wave_max(amax);
  const int sh = max(0, __builtin_amdgcn_frexp_expf(mx) - 15);
  const float down = __builtin_amdgcn_ldexpf(1.0f, -sh);
  const float zsc = __builtin_amdgcn_ldexpf(2.0f, sh);  // D -> log2 score units
#pragma unroll
  for (int k = 0; k < Gm::QPL; ++k) {
    const int h = g + 4 * k;
    const float bsum = row_sum(bp[k]);
    if (h < QB) {
      h8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qp[k][e] * down;
        const _Float16 xh = _Float16(x);
        hi[e] = xh;
        lo[e] = _Float16(x - float(xh));
      }
      *L.row(cb * 4 + cg, h) = hi;
      *L.row((((QB + h) / 16) * 4 + cb) * 4 + cg, (QB + h) % 16) = lo;
      if (j == 0) L.bias[h] = bsum;
    }
  }
  wave_lds_sync();
  h8 ak[Gm::NA][4];
#pragma unroll
  for (int a = 0; a < Gm::NA; ++a)
#pragma unroll
    for (int s = 0; s < 4; ++s) ak[a][s] = *L.row((a * 4 + s) * 4 + g, j);

  // ---- scores on the matrix cores, two tiles at a time into LDS
#pragma unroll
  for (int T = 0; T < Gm::KT; T += 2) {
    h8 b[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      codes_b(kc[T + u].x, b[u][0], b[u][1]);
      codes_b(kc[T + u].y, b[u][2], b[u][3]);
    }
    f4 d[2][Gm::NA];
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a)
#pragma unroll
      for (int u = 0; u < 2; ++u) d[u][a] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < Gm::NA; ++a)
#pragma unroll
        for (int u = 0; u < 2; ++u) d[u][a] = mfma16(ak[a][s], b[u][s], d[u][a]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f4* dst = reinterpret_cast<f4*>(&L.zs[(16 * (T + u) + j) * Gm::ZR + 4 * g]);
      if constexpr (Gm::NA == 2) {
        *dst = d[u][0] + d[u][1];
      } else {
        if (4 * g < 2 * QB) *dst = d[u][0];
      }
    }
  }
  wave_lds_sync();

  // ---- softmax over the page: lane takes token pairs, all QB heads
  float bias[QB];
#pragma unroll
  for (int h = 0; h < QB; h += 4) {
    const float4 b4 = *reinterpret_cast<const float4*>(&L.bias[h]);
    bias[h] = b4.x;
    if (h + 1 < QB) bias[h + 1] = b4.y;
    if (h + 2 < QB) bias[h + 2] = b4.z;
    if (h + 3 < QB) bias[h + 3] = b4.w;
  }
  float z[Gm::PPL][2][QB];
#pragma unroll
  for (int k = 0; k < Gm::PPL; ++k) {
    const int pi = lane + 64 * k;
    const bool pv = (Gm::NP % 64 == 0) || pi < Gm::NP;
    const int t0 = pair_token<G>(min(pi, Gm::NP - 1));
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int t = t0 + 2 * s2;
      const bool ok = pv && t < n_valid;
      float zr[Gm::ZR];
#pragma unroll
      for (int i = 0; i < Gm::ZR; i += 4) {
        const f4 v = *reinterpret_cast<const f4*>(&L.zs[t * Gm::ZR + i]);
        zr[i] = v[0]; zr[i + 1] = v[1]; zr[i + 2] = v[2]; zr[i + 3] = v[3];
      }
#pragma unroll
      for (int h = 0; h < QB; ++h) {
        const float v = (Gm::ZR == QB) ? zr[h] : zr[h] + zr[QB + h];
        z[k][s2][h] = ok ? fmaf(v, zsc, bias[h]) : -INFINITY;
      }
    }
  }
  float mh[QB];
#pragma unroll
  for (int h = 0; h < QB; ++h) {
    mh[h] = -INFINITY;
#pragma unroll
    for (int k = 0; k < Gm::PPL; ++k) mh[h] = fmaxf(mh[h], fmaxf(z[k][0][h], z[k][1][h]));
  }
  wave_max_n<QB>(mh);
  float alpha[QB], muse[QB];
  bool moved = false;
#pragma unroll
  for (int h = 0; h < QB; ++h) {
    const float mn = fmaxf(st.m[h], mh[h]);
    alpha[h] = (mn == st.m[h]) ? 1.f : (st.m[h] == -INFINITY ? 0.f : exp2_fast(st.m[h] - mn));
    moved |= (mn != st.m[h]);
    st.m[h] = mn;
    muse[h] = (mn == -INFINITY) ? 0.f : mn;
    st.l[h] *= alpha[h];
    st.vmin[h] *= alpha[h];
  }
  if (moved) {  // wave-uniform
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = row_pick<QB>(alpha, g, r);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[ct][r] *= ar[r];
  }
#pragma unroll
  for (int k = 0; k < Gm::PPL; ++k) {
    const int pi = lane + 64 * k;
    const bool pv = (Gm::NP % 64 == 0) || pi < Gm::NP;
    const int g2 = pi / (G / 8), rem = pi % (G / 8), kb = rem >> 2, p = rem & 3;
    float pp[2][QB];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const float mnt = lo_f(vm[k][s2]), sct = hi_f(vm[k][s2]);
#pragma unroll
      for (int h = 0; h < QB; ++h) {
        const float pr = exp2_fast(z[k][s2][h] - muse[h]);
        st.l[h] += pr;
        st.vmin[h] = fmaf(pr, mnt, st.vmin[h]);
        pp[s2][h] = pr * sct;  // p * scale_t <= 2^16 / 3 fits fp16
      }
    }
    uint32_t* prow = reinterpret_cast<uint32_t*>(L.ab + (kb * 4 + g2) * Gm::kBlk) + p;
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      const f16x2 two{_Float16(pp[0][h]), _Float16(pp[1][h])};
      if (pv) prow[4 * h] = __builtin_bit_cast(uint32_t, two);
    }
  }
  wave_lds_sync();

  // ---- values on the matrix cores
  h8 av[Gm::KB];
#pragma unroll
  for (int kb = 0; kb < Gm::KB; ++kb) av[kb] = *L.row(kb * 4 + g, j);
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
    for (int w = 0; w < Gm::VDW; ++w) {
      h8 b0, b1;
      codes_b(vc[ct][w], b0, b1);
      st.acc[ct] = mfma16(av[2 * w], b0, st.acc[ct]);
      st.acc[ct] = mfma16(av[2 * w + 1], b1, st.acc[ct]);
    }
  }
  wave_lds_sync();
}

// Work-group = 4 waves on one (sequence, KV head, split). Every wave holds the
// state of QB query heads, walks the split's fp16 tokens (its 16-token chunks,
// one head at a time) and then its pages (round-robin); the 4 states merge in
// LDS. More than QB heads per KV head run as several passes.
template <int G, int QB>
__global__ __launch_bounds__(256, (G * QB >= 2048) ? 1 : (G <= 128 && QB <= 4) ? 3 : 2) void decode_gqa_kernel(Arena a, const __half* __restrict__ q,
                                                         __half* __restrict__ out, int S,
                                                         HeadOrder order) {
  using Gm = Geo<G, QB>;
  __shared__ GqaLds<G, QB> lds_all[kWaves];
  __shared__ float mg_m[kWaves][QB], mg_l[kWaves][QB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  GqaLds<G, QB>& L = lds_all[wave];
  const int NQ = a.Hq / a.Hkv;
  const int s = blockIdx.x % S;
  const int bh = order.n ? int(order.bh[blockIdx.x]) : int(blockIdx.x / S);
  const int b = bh / a.Hkv, hk = bh % a.Hkv;

  const int32_t* ctr = counters(a, bh);
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  const int pc = min(a.P, a.G * nb);
  const Split sp = split_of(nb, pc + r_cnt, a.page_bytes, s, S);
  const int buf = nb & 1;
  const Fp16Src src{pool_k(a, buf, bh), pool_v(a, buf, bh), ring_k(a, bh), ring_v(a, bh), pc,
                    head, a.C};
  const float qscale = a.sm_scale * kLog2e;
  const uint8_t* pages = page_ptr(a, bh, 0);
  const int64_t PB = a.page_bytes;

  for (int q0 = 0; q0 < NQ; q0 += QB) {
    const int qh0 = hk * NQ + q0;
    const __half* qbase = q + (size_t(b) * a.Hq + qh0) * D;
    GqaState<QB> st;
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      st.m[h] = -INFINITY;
      st.l[h] = 0.f;
      st.vmin[h] = 0.f;
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f4{0.f, 0.f, 0.f, 0.f};

    // fp16 tokens: each chunk is loaded once per group of up to 4 heads; the
    // heads' states then enter the page state (which is still empty)
    constexpr int HG = QB < 4 ? QB : 4;
#pragma unroll 1
    for (int h0 = 0; h0 < QB; h0 += HG) {
      uint4 q8[HG];
      Fp16State fs[HG];
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        q8[i] = reinterpret_cast<const uint4*>(qbase + size_t(h0 + i) * D)[lane & 15];
        fs[i].m = -INFINITY;
        fs[i].l = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) fs[i].acc[e] = 0.f;
      }
      for (int ch = sp.t0 + wave * kF16Chunk; ch < sp.t1; ch += kWaves * kF16Chunk) {
        const int cnt = min(kF16Chunk, sp.t1 - ch);
        Fp16Rows rows;
        fp16_load(src, ch, cnt, rows, lane);
#pragma unroll
        for (int i = 0; i < HG; ++i) fp16_attend(rows, cnt, q8[i], qscale, fs[i], lane);
      }
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        const int h = h0 + i;
#pragma unroll
        for (int hh = 0; hh < QB; ++hh) {
          if (hh == h) {
            st.m[hh] = fs[i].m;
            st.l[hh] = fs[i].l;
          }
        }
        float4* f = reinterpret_cast<float4*>(&L.zs[(lane >> 4) * D + 8 * (lane & 15)]);
        f[0] = make_float4(fs[i].acc[0], fs[i].acc[1], fs[i].acc[2], fs[i].acc[3]);
        f[1] = make_float4(fs[i].acc[4], fs[i].acc[5], fs[i].acc[6], fs[i].acc[7]);
        wave_lds_sync();
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const int c = 16 * ct + j;
          const float v = (L.zs[c] + L.zs[D + c] + L.zs[2 * D + c] + L.zs[3 * D + c]) * 0.5f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r == h) st.acc[ct][r] = v;
        }
        wave_lds_sync();
      }
    }

    // the lane's query values for the q' step: heads g + 4k, channels
    // 8j + kPerm(slot)
    float qs[Gm::QPL][8];
#pragma unroll
    for (int k = 0; k < Gm::QPL; ++k) {
      const int h = g + 4 * k;
      if (h < QB) {
        const uint4 q8 = *reinterpret_cast<const uint4*>(qbase + size_t(h) * D + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = kPerm(e);
          const uint32_t w = dw(q8, c >> 1);
          qs[k][e] = ((c & 1) ? hi_f(w) : lo_f(w)) * qscale;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[k][e] = 0.f;
      }
    }

    // pages, each wave every 4th
    for (int u = sp.p0 + wave; u < sp.p1; u += kWaves) {
      prio_by_work_left((sp.p1 - u + kWaves - 1) / kWaves);
      GqaPage<G> pr;
      gqa_load<G>(pr, pages + size_t(u) * PB, lane);
      gqa_page<G, QB>(pr, page_nvalid(a.G, a.P, u), qs, L, st, lane);
    }

    // this wave's state -> LDS: fin[h][c] = sum p' c + sum p min = 2 acc + vmin
    float vt[QB];
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      const float lt = wave_sum(st.l[h]);
      vt[h] = wave_sum(st.vmin[h]);
      if (lane == 0) {
        mg_m[wave][h] = st.m[h];
        mg_l[wave][h] = lt;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      const float v = row_pick<QB>(vt, g, r);
      if (h < QB) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) L.zs[h * D + 16 * ct + j] = fmaf(st.acc[ct][r], 2.0f, v);
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < QB * D; x += blockDim.x) {
      const int h = x / D, c = x % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mg_m[w][h]);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = (mg_m[w][h] == -INFINITY) ? 0.f : exp2f(mg_m[w][h] - M);
        Ls = fmaf(mg_l[w][h], f, Ls);
        A = fmaf(lds_all[w].zs[h * D + c], f, A);
      }
      const int qh = qh0 + h;
      if (S == 1) {
        out[(size_t(b) * a.Hq + qh) * D + c] = __float2half_rn(A / Ls);
      } else {
        float* part = partial_ptr(a, b, qh, s);
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

template <int G>
hipError_t launch_g(const Arena& a, const __half* q, __half* out, int S, const HeadOrder& order,
                    hipStream_t s) {
  const int NQ = a.Hq / a.Hkv;
  const dim3 grid(unsigned(a.B) * a.Hkv * S), block(64 * kWaves);
  if (NQ % 16 == 0) {
    hipLaunchKernelGGL((decode_gqa_kernel<G, 16>), grid, block, 0, s, a, q, out, S, order);
  } else if (NQ % 8 == 0) {
    hipLaunchKernelGGL((decode_gqa_kernel<G, 8>), grid, block, 0, s, a, q, out, S, order);
  } else if (NQ % 4 == 0) {
    hipLaunchKernelGGL((decode_gqa_kernel<G, 4>), grid, block, 0, s, a, q, out, S, order);
  } else if (NQ == 2) {
    hipLaunchKernelGGL((decode_gqa_kernel<G, 2>), grid, block, 0, s, a, q, out, S, order);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G>
int wgs_g(const Arena& a) {
  const int NQ = a.Hq / a.Hkv;
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  const int bs = 64 * kWaves;
  if (NQ % 16 == 0) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 16>, bs, 0);
  else if (NQ % 8 == 0) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 8>, bs, 0);
  else if (NQ % 4 == 0) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 4>, bs, 0);
  else if (NQ == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 2>, bs, 0);
  return e == hipSuccess ? n : 0;
}

}  // namespace

int decode_gqa_wgs_per_cu(const Arena& a) {
  switch (a.G) {
    case 64: return wgs_g<64>(a);
    case 128: return wgs_g<128>(a);
    case 256: return wgs_g<256>(a);
    default: return 0;
  }
}

hipError_t launch_decode_gqa(const Arena& a, const void* q, void* out, int S,
                             const HeadOrder& order, hipStream_t s) {
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  switch (a.G) {
    case 64: return launch_g<64>(a, qh, oh, S, order, s);
    case 128: return launch_g<128>(a, qh, oh, S, order, s);
    case 256: return launch_g<256>(a, qh, oh, S, order, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ott
