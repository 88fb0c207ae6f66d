// Decoding stage for grouped query heads (several query heads per KV head) on
// the gfx950 fp8 x fp4 matrix cores.
//
// Same computation as the one-head kernel ([Blog] zijie-tian.site summary,
// section 3.3 flowchart; [Abs] sciencestack.ai, Figure 2 top): scores of the
// quantized Keys, the window Keys and the pool Keys go under one softmax and
// the weights multiply the matching Values. The query heads that share a page
// make both products over it small dense contractions:
//
//   scores  z[h][t] = bias[h] + sum_c q'[h][c] * kcode[t][c]
//   values  o[h][c] += sum_t p'[h][t] * vcode[c][t]
//
// with q'[h][c] = qs[h][c] * scale_c and p'[h][t] = p[h][t] * scale_t. Both run
// on v_mfma_scale_f32_16x16x128_f8f6f4 (operand layouts and the exactness of
// fixed-point digit rows in ott_mx.h): a group of 4 query heads fills the 16 A
// rows with 4 digit rows per head (row 4h + k = digit k of head h, each row
// with its own E8M0 scale), and the 2-bit codes are the B operand as FP4.
// Result row 4h + k then sits in lane group h, so every lane group owns one
// head of the group: its scores, its softmax state and its value sums.
//
// Token order of the score tiles. K tile T holds the 16 consecutive tokens
// 16T..16T+15; column j is token 16T + mx_item(j), the one at position j of
// the tile's 16-slot stretch of the value operand. So each load of a tile's
// codes reads whole cache lines that no other load of the page touches. A
// lane's scores then sit at one slot in each 16-slot stretch; a 4 x 4 byte
// transpose inside each quad of lanes turns every 4 tiles of a digit row of p'
// into one 4-byte LDS write per lane.
#include "ott_decode_common.h"
#include "ott_mx.h"

namespace ott {
namespace {
using namespace dev;
using namespace dec;

template <int G>
struct Gx {
  static constexpr int NB = (G + 127) / 128;         // value k-blocks of 128 slots
  static constexpr int NT = G / 16;                  // score tiles
  static constexpr int RS = 144;                     // LDS bytes per A row (128 + pad)
  static constexpr int ABLK = 16 * RS;               // one A operand block
};

// token of score tile T, column j (j < 16)
__device__ __forceinline__ int gx_token(int T, int j) { return 16 * T + mx_item(j); }

// 4 x 4 byte transpose in each quad of lanes: byte b of lane 4m + i's result
// is byte i of lane 4m + b's x. Two exchanges: 16-bit halves with lane i ^ 2,
// then bytes with lane i ^ 1 (v_perm_b32 picks bytes 0-3 from its second
// operand and 4-7 from its first).
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t x, int lane) {
  const int i = lane & 3;
  const uint32_t p = uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kQuadSwap2, 0xF, 0xF, false));
  const uint32_t e = __builtin_amdgcn_perm(p, x, (i & 2) ? 0x03020706u : 0x05040100u);
  const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(e), kQuadSwap1, 0xF, 0xF, false));
  return __builtin_amdgcn_perm(o, e, (i & 1) ? 0x03070105u : 0x06020400u);
}

// The part of a page one lane reads from memory.
template <int G>
struct GxPage {
  static constexpr int NT = Gx<G>::NT, NB = Gx<G>::NB;
  uint4 km[2];         // K (min, scale) of channels 8(lane&15)..+7
  uint2 kc[NT];        // K codes: tile T, token gx_token(T, lane&15), channels 32g..32g+31
  uint32_t vm[NT];     // V (min, scale) of the lane's tokens
  uint2 vc[8][NB];     // V codes: channel 16C + (lane&15), block h: slots 128h + 32g..+31
                       // (G = 256: slots 64g + 32h..+31, one 16-byte load for both)
};

template <int G>
__device__ __forceinline__ void gx_load(GxPage<G>& r, const uint8_t* __restrict__ pg, int lane) {
  constexpr int NT = Gx<G>::NT, NB = Gx<G>::NB;
  const int j = lane & 15, g = lane >> 4;
  r.km[0] = ld_nt4(pg + kmeta_off(G) + 32 * j);
  r.km[1] = ld_nt4(pg + kmeta_off(G) + 32 * j + 16);
#pragma unroll
  for (int T = 0; T < NT; ++T) r.kc[T] = ld_nt2(pg + gx_token(T, j) * (D / 4) + 8 * g);
#pragma unroll
  for (int T = 0; T < NT; ++T) r.vm[T] = ld_nt1(pg + vmeta_off(G) + 4 * gx_token(T, j));
#pragma unroll
  for (int C = 0; C < 8; ++C)
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const uint8_t* row = pg + vcode_off(G) + (16 * C + j) * (G / 4);
      if constexpr (G == 256) {
        if (h == 0) {
          const uint4 x = ld_nt4(row + 16 * g);
          r.vc[C][0] = make_uint2(x.x, x.y);
          r.vc[C][1] = make_uint2(x.z, x.w);
        }
      } else if constexpr (G == 128) {
        r.vc[C][h] = ld_nt2(row + 8 * g);
      } else {  // a 16-byte row: lane groups 2 and 3 have no slots
        r.vc[C][h] = ld_nt2(row + 8 * (g & 1));
        if (g >= 2) r.vc[C][h] = make_uint2(0u, 0u);
      }
    }
}

// Online softmax state of one wave for NA groups of 4 query heads; lane group
// g holds head 4a + g of group a.
template <int NA>
struct GxState {
  float m[NA];       // running max (uniform in the lane group)
  float l[NA];       // this lane's share of the running sum
  float vmin[NA];    // this lane's share of sum p_t min_t
  f32x4v acc[NA][8]; // digit-row sums: channel 16C + (lane&15), rows = the head's digits
};

// A operand of row (lane & 15): logical k 16g..16g+15 and 64+16g..64+16g+15
template <int G>
__device__ __forceinline__ i32x8 gx_a(const uint8_t* blk, int lane) {
  const uint8_t* r = blk + Gx<G>::RS * (lane & 15) + 16 * (lane >> 4);
  const uint4 lo = *reinterpret_cast<const uint4*>(r);
  const uint4 hi = *reinterpret_cast<const uint4*>(r + 64);
  i32x8 a;
  a[0] = int(lo.x); a[1] = int(lo.y); a[2] = int(lo.z); a[3] = int(lo.w);
  a[4] = int(hi.x); a[5] = int(hi.y); a[6] = int(hi.z); a[7] = int(hi.w);
  return a;
}

// Scale register of lane l: row l & 15 = digit (l & 3) of head (l & 15) >> 2,
// whose exponent e lives in lane group (l & 15) >> 2; times 2 for code/2.
// One backward permute fetches it from lane 16 ((l & 15) >> 2) (byte address
// four times the lane).
__device__ __forceinline__ int gx_scale(int e, int lane) {
  const int eh = __builtin_amdgcn_ds_bpermute((lane & 12) << 4, e);
  return 124 + eh - 5 * (lane & 3);
}

// One fixed-point digit of r (r scaled so that |r| < 16 at the first digit):
// the digit, with r left as 32 x the rest, as mx_digits does for all four.
__device__ __forceinline__ float gx_digit(float& r) {
  const float d = __builtin_rintf(r);
  r = (r - d) * 32.0f;
  return d;
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

template <int G, int NA>
struct alignas(16) GxLds {
  // q' operands (NA blocks), then p' operands (NA x NB blocks); reused for the
  // fp16 fold and the final state
  uint8_t ab[NA * (1 + Gx<G>::NB) * Gx<G>::ABLK];
  __device__ __forceinline__ uint8_t* qa(int a) { return ab + a * Gx<G>::ABLK; }
  __device__ __forceinline__ uint8_t* pa(int a, int h) {
    return ab + (NA + a * Gx<G>::NB + h) * Gx<G>::ABLK;
  }
  __device__ __forceinline__ float* f(int i) { return reinterpret_cast<float*>(ab) + i; }
};

template <int G, int NA>
__device__ __forceinline__ void gx_page(const GxPage<G>& r, int n_valid, const float (&qs)[NA][8],
                                        GxLds<G, NA>& L, GxState<NA>& st, int lane) {
  constexpr int NT = Gx<G>::NT, NB = Gx<G>::NB, RS = Gx<G>::RS;
  const int j = lane & 15, g = lane >> 4;

  // ---- q' = qs scale_c for head g of each group, channels 8j..8j+7, as digits
  float mnv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mnv[i] = lo_f(dw(r.km[i >> 2], i & 3));
  // channel 8j + i sits at logical k = base + (i >> 1) + 8 (i & 1)
  const int base = 32 * (j >> 2) + 16 * ((j >> 1) & 1) + 4 * (j & 1);
  float bias[NA];
  int sq[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    float qp[8], b = 0.f, amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qp[i] = mul_hi_f(qs[a][i], dw(r.km[i >> 2], i & 3));
      b = fmaf(qs[a][i], mnv[i], b);
      amax = fmaxf(amax, fabsf(qp[i]));
    }
    bias[a] = row_sum(b);
    const int eq = mx_exp(row_max_nonneg(amax));
    // digit rows one at a time (see mx_digits): r holds what is left
#pragma unroll
    for (int i = 0; i < 8; ++i) qp[i] = __builtin_amdgcn_ldexpf(qp[i], 4 - eq);
    uint8_t* blk = L.qa(a);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = gx_digit(qp[i]);
      uint8_t* row = blk + RS * (4 * g + k);
      *reinterpret_cast<uint32_t*>(row + base) = pack4_fp8(d[0], d[2], d[4], d[6]);
      *reinterpret_cast<uint32_t*>(row + base + 8) = pack4_fp8(d[1], d[3], d[5], d[7]);
    }
    sq[a] = gx_scale(eq, lane);
  }
  wave_lds_sync();

  // ---- scores on the matrix cores
  float z[NA][NT];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const i32x8 aq = gx_a<G>(L.qa(a), lane);
    if constexpr (NT <= 8) {
      // all tiles issued before any result is read, so the products overlap
      f32x4v zr[NT];
#pragma unroll
      for (int T = 0; T < NT; ++T)
        zr[T] = mx_mfma<0>(aq, mx_b(r.kc[T]), f32x4v{0.f, 0.f, 0.f, 0.f}, sq[a]);
#pragma unroll
      for (int T = 0; T < NT; ++T)
        z[a][T] = bias[a] + ((zr[T][0] + zr[T][1]) + (zr[T][2] + zr[T][3]));
    } else {  // G = 256: 16 live results would not fit beside the page
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        const f32x4v zr = mx_mfma<0>(aq, mx_b(r.kc[T]), f32x4v{0.f, 0.f, 0.f, 0.f}, sq[a]);
        z[a][T] = bias[a] + ((zr[0] + zr[1]) + (zr[2] + zr[3]));
      }
    }
  }
  if (n_valid < G) {
#pragma unroll
    for (int T = 0; T < NT; ++T)
      if (gx_token(T, j) >= n_valid)
#pragma unroll
        for (int a = 0; a < NA; ++a) z[a][T] = -INFINITY;
  }

  // ---- softmax: head 4a + g over the lane group's 16 lanes
  bool moved = false;
  float alpha[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    float mx = z[a][0];
#pragma unroll
    for (int T = 1; T < NT; ++T) mx = fmaxf(mx, z[a][T]);
    mx = row_max_ordered(mx);
    const float mn = fmaxf(st.m[a], mx);
    alpha[a] = (mn == st.m[a]) ? 1.f : (st.m[a] == -INFINITY ? 0.f : exp2_fast(st.m[a] - mn));
    moved |= (mn != st.m[a]);
    st.m[a] = mn;
    st.l[a] *= alpha[a];
    st.vmin[a] *= alpha[a];
  }
  if (__ballot(moved) != 0) {  // wave-uniform
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int C = 0; C < 8; ++C) st.acc[a][C] *= alpha[a];
  }
  int sp[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    // a page without members leaves m at -inf only if nothing came before;
    // its weights are then 0 (m = -inf -> use 0 as the reference)
    const float mref = (st.m[a] == -INFINITY) ? 0.f : st.m[a];
    float pp[NT], pmax = 0.f;
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const float p = exp2_fast(z[a][T] - mref);
      st.l[a] += p;
      st.vmin[a] = fmaf(p, lo_f(r.vm[T]), st.vmin[a]);
      pp[T] = mul_hi_f(p, r.vm[T]);
      pmax = fmaxf(pmax, pp[T]);
    }
    const int ep = mx_exp(row_max_nonneg(pmax));
#pragma unroll
    for (int T = 0; T < NT; ++T) pp[T] = __builtin_amdgcn_ldexpf(pp[T], 4 - ep);
    // tiles 4u..4u+3: slots 4(j >> 2) + 0..3 of tile T's 16-slot stretch of a
    // digit row come from lanes 4(j >> 2) + 0..3; lane j writes tile
    // T = 4u + (j & 3). The stretch is 16T of block 0 (G <= 128); at G = 256,
    // 32(T / 4) + 16(T % 2) of block (T / 2) % 2.
    const int tq = j & 3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int u = 0; u < NT / 4; ++u) {
        const int T0 = 4 * u;
        const float d0 = gx_digit(pp[T0]), d1 = gx_digit(pp[T0 + 1]);
        const float d2 = gx_digit(pp[T0 + 2]), d3 = gx_digit(pp[T0 + 3]);
        const uint32_t w = quad_transpose_bytes(pack4_fp8(d0, d1, d2, d3), lane);
        uint8_t* blk = G == 256 ? L.pa(a, tq >> 1) + 32 * u + 16 * (tq & 1)
                                : L.pa(a, 0) + 16 * (4 * u + tq);
        *reinterpret_cast<uint32_t*>(blk + RS * (4 * g + k) + 4 * (j >> 2)) = w;
      }
    }
    sp[a] = gx_scale(ep, lane);
  }
  wave_lds_sync();

  // ---- values on the matrix cores
#pragma unroll
  for (int a = 0; a < NA; ++a) {
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      i32x8 ap = gx_a<G>(L.pa(a, h), lane);
      if constexpr (G < 128) {  // logical k >= 64 has no slots (and no written bytes)
        ap[4] = 0; ap[5] = 0; ap[6] = 0; ap[7] = 0;
      }
#pragma unroll
      for (int C = 0; C < 8; ++C) st.acc[a][C] = mx_mfma<0>(ap, mx_b(r.vc[C][h]), st.acc[a][C], sp[a]);
    }
  }
  wave_lds_sync();
}

// Work-group = 4 waves on one (sequence, KV head, split). Each pass serves
// 4 NA query heads of the KV head: every wave walks its share of the split's
// fp16 tokens (16-token chunks, one load per group of 4 heads), folds them into
// its state, then walks its pages (round-robin); the 4 wave states merge in
// LDS. Heads past the KV head's last (a padded group) get a zero query and are
// not written.
// kStep: a fused step's decode (the new token, counter advances, the store).
template <int G, int NA, bool kStep>
__global__ __launch_bounds__(256, NA == 1 ? (G <= 128 ? 3 : 2) : 1) void decode_gqa_kernel(
    Arena a, const __half* __restrict__ q, __half* __restrict__ out, int S, HeadOrder order,
    StepArgs step) {
  constexpr int QB = 4 * NA;
  __shared__ GxLds<G, NA> lds_all[kWaves];
  __shared__ float mg_m[kWaves][QB], mg_l[kWaves][QB];
  __shared__ uint32_t mg_last;
  // The prologue (counters, query rows, fp16 chunks) is a chain of dependent
  // loads: at the top priority, a work-group that starts beside others
  // already in their page loops is not held back by them.
  __builtin_amdgcn_s_setprio(3);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  GxLds<G, NA>& L = lds_all[wave];
  const int NQ = a.Hq / a.Hkv;
  const int s = blockIdx.x % S;
  const int bh = order.n ? int(order.bh[blockIdx.x]) : int(blockIdx.x / S);
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  // Query row h of the KV head's group, the lane's 16 bytes (channels
  // 8(lane & 15)..+7); zero past the group's last head.
  const __half* qkv = q + (size_t(b) * a.Hq + size_t(hk) * NQ) * D;
  auto q_row = [&](int h) {
    return h < NQ ? reinterpret_cast<const uint4*>(qkv + size_t(h) * D)[j] : make_uint4(0u, 0u, 0u, 0u);
  };
  // The page loop's query values (head 4x + g, channels 8j..8j+7) of the first
  // pass are read before the counters, so the two reads wait together.
  uint4 mine_first[NA];
#pragma unroll
  for (int x = 0; x < NA; ++x) mine_first[x] = q_row(4 * x + g);

  const HeadCtr hc = head_counters<kStep>(a, step, b, bh);
  const int r_cnt = hc.r_cnt, head = hc.head, nb = hc.nb;
  const int pc = min(a.P, a.G * nb);
  const int n_new = kStep ? 1 : 0;  // a fused step's new token, after the window
  const Split sp = split_of(nb, pc + r_cnt + n_new, s, S);
  const int buf = nb & 1;
  const Fp16Src base_src{pool_k(a, buf, bh), pool_v(a, buf, bh), ring_k(a, bh), ring_v(a, bh), pc,
                         head, a.C};
  const auto src = [&] {
    if constexpr (kStep)
      return Fp16StepSrc{base_src, pc + r_cnt, step.k + size_t(bh) * D, step.v + size_t(bh) * D};
    else
      return base_src;
  }();
  const float qscale = a.sm_scale * kLog2e;
  const uint8_t* pages = page_ptr(a, bh, 0);
  const int64_t PB = a.page_bytes;

  for (int q0 = 0; q0 < NQ; q0 += QB) {
    const int qh0 = hk * NQ + q0;
    GxState<NA> st;
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      st.m[x] = -INFINITY;
      st.l[x] = 0.f;
      st.vmin[x] = 0.f;
#pragma unroll
      for (int C = 0; C < 8; ++C) st.acc[x][C] = f32x4v{0.f, 0.f, 0.f, 0.f};
    }

    // fp16 tokens: each chunk is loaded once per group of 4 heads; the heads'
    // states then become the (still empty) page states, the accumulator in
    // digit row 0
    float qs[NA][8];  // the lane's query values for the q' step: head 4x + g, channels 8j..8j+7
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      {
        const uint4 mine = q0 == 0 ? mine_first[x] : q_row(q0 + 4 * x + g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w = dw(mine, i >> 1);
          qs[x][i] = ((i & 1) ? hi_f(w) : lo_f(w)) * qscale;
        }
      }
      uint4 q8[4];  // the group's four rows, for the fp16 tokens
#pragma unroll
      for (int i = 0; i < 4; ++i) q8[i] = q_row(q0 + 4 * x + i);
      Fp16State fs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fs[i].m = -INFINITY;
        fs[i].l = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) fs[i].acc[e] = 0.f;
      }
      for (int ch = first_chunk(sp, wave); ch < sp.t1; ch += kWaves * kF16Chunk) {
        const int cnt = min(kF16Chunk, sp.t1 - ch);
        Fp16Rows rows;
        fp16_load(src, ch, cnt, rows, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) fp16_attend(rows, cnt, q8[i], qscale, fs[i], lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lt = wave_sum(fs[i].l);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // the four token rows of each channel add up
          f32x2 p = swap16(fs[i].acc[e]);
          const float y = p.x + p.y;
          p = swap32(y);
          v[e] = p.x + p.y;
        }
        float* f = L.f(0);
        if (lane < 16) {
          reinterpret_cast<float4*>(f + 8 * lane)[0] = make_float4(v[0], v[1], v[2], v[3]);
          reinterpret_cast<float4*>(f + 8 * lane)[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        wave_lds_sync();
        if (g == i) {
          st.m[x] = fs[i].m;
          st.l[x] = (j == 0) ? lt : 0.f;
#pragma unroll
          for (int C = 0; C < 8; ++C) st.acc[x][C][0] = f[16 * C + j];
        }
        wave_lds_sync();
      }
    }


    // pages, each wave every 4th
    for (int u = sp.p0 + wave; u < sp.p1; u += kWaves) {
      prio_by_work_left((sp.p1 - u + kWaves - 1) / kWaves);
      GxPage<G> pr;
      gx_load<G>(pr, pages + size_t(u) * PB, lane);
      gx_page<G, NA>(pr, page_nvalid(a.G, a.P, u), qs, L, st, lane);
    }

    // this wave's state -> LDS: fin[h][c] = sum of the digit rows + sum p min
    float* fin = L.f(0);
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      const float lt = row_sum(st.l[x]);
      const float vt = row_sum(st.vmin[x]);
      const int h = 4 * x + g;
      if (j == 0) {
        mg_m[wave][h] = st.m[x];
        mg_l[wave][h] = lt;
      }
#pragma unroll
      for (int C = 0; C < 8; ++C) {
        const f32x4v v = st.acc[x][C];
        fin[h * D + 16 * C + j] = ((v[0] + v[1]) + (v[2] + v[3])) + vt;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < QB * D; x += blockDim.x) {
      const int h = x / D, c = x % D;
      if (q0 + h >= NQ) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mg_m[w][h]);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = (mg_m[w][h] == -INFINITY) ? 0.f : exp2f(mg_m[w][h] - M);
        Ls = fmaf(mg_l[w][h], f, Ls);
        A = fmaf(lds_all[w].f(0)[h * D + c], f, A);
      }
      const int qh = qh0 + h;
      if (S == 1) {
        out[(size_t(b) * a.Hq + qh) * D + c] = __float2half_rn(A / Ls);
      } else {
        float* part = partial_ptr(a, b, qh, s);
        st_coherent(part + 2 + c, A);
        if (c == 0) {
          st_coherent(part, M);
          st_coherent(part + 1, Ls);
        }
      }
    }
    __syncthreads();
  }
  // a fused step's new row (its loads go out before the split arrival's wait)
  uint4 piece{};
  if (kStep && threadIdx.x < 32) piece = step_row_piece(step, bh, threadIdx.x);
  // a fused step with one split: this work-group is the head's only reader of
  // its counters, so it stores the new token and the counters itself
  if (kStep && S == 1 && threadIdx.x < 32) step_store(a, bh, hc, threadIdx.x, piece);
  // several splits: the last one to finish merges them for every query head
  // of the KV head (and is the step's writer: every split has read the
  // counters and the window by then)
  if (S > 1 && last_split(a, bh, S, &mg_last)) {
    // two outputs per thread and round, their loads in flight together
    constexpr int kT = 64 * kWaves;
    for (int x = threadIdx.x; x < NQ * D; x += 2 * kT) {
      const int x1 = min(x + kT, NQ * D - 1);  // (a repeat of x's row when past the end)
      const float* const ps[2] = {partial_ptr(a, b, hk * NQ + x / D, 0),
                                  partial_ptr(a, b, hk * NQ + x1 / D, 0)};
      const int cs[2] = {x % D, x1 % D};
      float o[2];
      merge_partials_n<true, 2>(ps, S, cs, o);
      out[(size_t(b) * a.Hq + hk * NQ) * D + x] = __float2half_rn(o[0]);
      if (x + kT < NQ * D) out[(size_t(b) * a.Hq + hk * NQ) * D + x1] = __float2half_rn(o[1]);
    }
    if (kStep && threadIdx.x < 32) step_store(a, bh, hc, threadIdx.x, piece);
    if (threadIdx.x == 0) reset_ticket(a, bh);
  }
}

template <int G>
hipError_t launch_g(const Arena& a, const __half* q, __half* out, int S, const HeadOrder& order,
                    const StepArgs& step, hipStream_t s) {
  const int NQ = a.Hq / a.Hkv;
  const dim3 grid(unsigned(a.B) * a.Hkv * S), block(64 * kWaves);
  if (step.k) {
    if (NQ % 8 == 0)
      hipLaunchKernelGGL((decode_gqa_kernel<G, 2, true>), grid, block, 0, s, a, q, out, S, order, step);
    else
      hipLaunchKernelGGL((decode_gqa_kernel<G, 1, true>), grid, block, 0, s, a, q, out, S, order, step);
  } else {
    if (NQ % 8 == 0)
      hipLaunchKernelGGL((decode_gqa_kernel<G, 2, false>), grid, block, 0, s, a, q, out, S, order, step);
    else
      hipLaunchKernelGGL((decode_gqa_kernel<G, 1, false>), grid, block, 0, s, a, q, out, S, order, step);
  }
  return hipGetLastError();
}

template <int G>
int wgs_g(const Arena& a) {
  const int NQ = a.Hq / a.Hkv;
  int n = 0;
  const int bs = 64 * kWaves;
  const hipError_t e =
      (NQ % 8 == 0) ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 2, false>, bs, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_gqa_kernel<G, 1, false>, bs, 0);
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
                             const HeadOrder& order, const StepArgs& step, hipStream_t s) {
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  switch (a.G) {
    case 64: return launch_g<64>(a, qh, oh, S, order, step, s);
    case 128: return launch_g<128>(a, qh, oh, S, order, step, s);
    case 256: return launch_g<256>(a, qh, oh, S, order, step, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ott
