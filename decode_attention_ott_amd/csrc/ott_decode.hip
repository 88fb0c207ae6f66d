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
// A split is an even share of one (sequence, KV head)'s pages and an even
// share of its fp16 tokens (pool first, then the window). With one
// split the work-group writes the output; otherwise every split writes its
// partial state and takes a ticket, and the head's last split to arrive merges
// all of them in the same launch (no second kernel, no launch gap).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ott_decode_common.h"
#include "ott_mx.h"

namespace ott {
namespace {
using namespace dev;
using namespace dec;

// Online softmax state of one wave (scores in log2 units) while it walks
// quantized pages.
struct WaveState {
  float m;        // running max (wave-uniform)
  float l;        // this lane's share of the running sum of weights
  float vmin;     // this lane's share of sum p_t * min_t over quantized tokens
  // acc[0..3]: digit-row partial sums of channel 16(lane>>4) + (lane&15);
  // acc[4..7]: those of that channel + 64
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
// quantized pages on the matrix cores
// ---------------------------------------------------------------------------
// The page products run on the fp8 x fp4 matrix cores (helpers and exactness
// argument in ott_mx.h).
//
// Rows: A holds the 4 digit rows of the page four times (rows 4i..4i+3). The
// scale register packs one byte per replica; byte i is the real scale for
// replica i and 0 (2^-127) for the others, and tile T runs with op_sel T % 4.
// Tiles 0..3 accumulate into one result and 4..7 into another, so lane group g
// ends with exactly its own tiles g and g+4 (the masked products add at most
// 2^-110 in total).

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


// Lane (j, g) of a page of G tokens: K tiles T = 0..G/16-1 (token 16T + j);
// the lane's tokens are slots 16g + j + 64i, i < G/64; V k-blocks of 128 slots
// (G = 64 leaves the upper half of the one block empty). At G = 256 block h
// holds the 32-slot stretches 64g' + 32h + 0..31 (g' = 0..3), so that a lane
// reads 16 contiguous bytes of a channel's 64-byte code row for both blocks
// and no cache line is requested by two loads.
template <int G>
struct MxPage {
  static constexpr int NT = G / 16;              // K tiles
  static constexpr int NZ = G / 64;              // tokens per lane
  static constexpr int NB = (G + 127) / 128;     // V k-blocks
  uint2 kc[NT];     // K tile T: token 16T + j, channel items 32g..32g+31
  uint2 vc[8][NB];  // V tile C, block h: channel 16C + j, slots 128h + 32g + 0..31
                    // (G = 256: slots 64g + 32h + 0..31)
  uint32_t km[2];   // K (min, scale) of the lane's channels c0 and c0 + 2
  uint32_t vm[NZ];  // V (min, scale) of the lane's slots
};

template <int G>
__device__ __forceinline__ void mx_load(MxPage<G>& r, const uint8_t* __restrict__ pg, int lane,
                                        int c0) {
  using P = MxPage<G>;
  const int j = lane & 15, g = lane >> 4;
  r.km[0] = ld_nt1(pg + kmeta_off(G) + 4 * c0);
  r.km[1] = ld_nt1(pg + kmeta_off(G) + 4 * (c0 + 2));
#pragma unroll
  for (int T = 0; T < P::NT; ++T) r.kc[T] = ld_nt2(pg + (16 * T + j) * (D / 4) + 8 * g);
#pragma unroll
  for (int i = 0; i < P::NZ; ++i) r.vm[i] = ld_nt1(pg + vmeta_off(G) + 4 * (16 * g + j + 64 * i));
#pragma unroll
  for (int C = 0; C < 8; ++C)
#pragma unroll
    for (int h = 0; h < P::NB; ++h) {
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

// One page; the state's acc[0..3] and acc[4..7] are the digit-row sums of the
// lane's channels 16g + j and 64 + 16g + j (full units).
template <int G>
__device__ __forceinline__ void mx_page(const MxPage<G>& r, int n_valid, float qs0, float qs1,
                                        uint8_t* qa, uint8_t* pa, WaveState& st, int lane) {
  using P = MxPage<G>;
  constexpr int NZ = P::NZ, NB = P::NB;
  const int j = lane & 15, g = lane >> 4;
  // ---- scores: q'_c = q_c scale_c as digits, bias = sum_c q_c min_c
  const float qp0 = mul_hi_f(qs0, r.km[0]), qp1 = mul_hi_f(qs1, r.km[1]);
  const float bias = wave_sum(fmaf(qs0, lo_f(r.km[0]), qs1 * lo_f(r.km[1])));
  const int eq = mx_exp(wave_max_nonneg(fmaxf(fabsf(qp0), fabsf(qp1))));
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
  f32x4v zr[NZ];
#pragma unroll
  for (int i = 0; i < NZ; ++i) zr[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NZ; ++i) zr[i] = mx_mfma<0>(aq, mx_b(r.kc[4 * i + 0]), zr[i], sq);
#pragma unroll
  for (int i = 0; i < NZ; ++i) zr[i] = mx_mfma<1>(aq, mx_b(r.kc[4 * i + 1]), zr[i], sq);
#pragma unroll
  for (int i = 0; i < NZ; ++i) zr[i] = mx_mfma<2>(aq, mx_b(r.kc[4 * i + 2]), zr[i], sq);
#pragma unroll
  for (int i = 0; i < NZ; ++i) zr[i] = mx_mfma<3>(aq, mx_b(r.kc[4 * i + 3]), zr[i], sq);
  const int t0 = 16 * g + j;
  float z[NZ];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NZ; ++i) {
    z[i] = bias + ((zr[i][0] + zr[i][1]) + (zr[i][2] + zr[i][3]));
    if (n_valid < G && t0 + 64 * i >= n_valid) z[i] = -INFINITY;  // a short page
    mx = fmaxf(mx, z[i]);
  }
  mx = wave_max_ordered(mx);
  if (mx == -INFINITY) return;  // a page without members
  rescale_q(st, fmaxf(st.m, mx));
  // ---- values: p'_t = p_t scale_t as digits
  float pp[NZ];
  float pmax = 0.f;
#pragma unroll
  for (int i = 0; i < NZ; ++i) {
    const float p = exp2_fast(z[i] - st.m);
    st.l += p;
    st.vmin = fmaf(p, lo_f(r.vm[i]), st.vmin);
    pp[i] = mul_hi_f(p, r.vm[i]);
    pmax = fmaxf(pmax, pp[i]);
  }
  const int ep = mx_exp(wave_max_nonneg(pmax));
  {
    // slot t0 + 64i sits in block i/2 at mx_k(t0) + 64 (i & 1); at G = 256 in
    // block t0 / 32 at mx_k(t0 % 32) + 32i
    constexpr int kStep = G == 256 ? 32 : 64;
#pragma unroll
    for (int i = 0; i < NZ; i += 2) {
      float d0[4], d1[4];
      mx_digits(pp[i], ep, d0);
      if (i + 1 < NZ) mx_digits(pp[i + 1], ep, d1);
      uint8_t* blk = G == 256 ? pa + 512 * (t0 >> 5) + mx_k(t0 & 31) + 32 * i
                              : pa + 512 * (i / 2) + mx_k(t0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = uint32_t(
            __builtin_amdgcn_cvt_pk_fp8_f32(d0[k], i + 1 < NZ ? d1[k] : 0.f, 0, false));
        blk[128 * k] = uint8_t(w);
        if (i + 1 < NZ) blk[128 * k + kStep] = uint8_t(w >> 8);
      }
    }
  }
  wave_lds_sync();
  i32x8 ap[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) ap[h] = mx_a(pa + 512 * h, lane);
  if constexpr (G < 128) {  // logical k >= 64 has no slots
    ap[0][4] = 0; ap[0][5] = 0; ap[0][6] = 0; ap[0][7] = 0;
  }
  const int sp = mx_scale(ep, lane);
  f32x4v va = {st.acc[0], st.acc[1], st.acc[2], st.acc[3]};
  f32x4v vb = {st.acc[4], st.acc[5], st.acc[6], st.acc[7]};
#pragma unroll
  for (int h = 0; h < NB; ++h) {
    va = mx_mfma<0>(ap[h], mx_b(r.vc[0][h]), va, sp);
    vb = mx_mfma<0>(ap[h], mx_b(r.vc[4][h]), vb, sp);
    va = mx_mfma<1>(ap[h], mx_b(r.vc[1][h]), va, sp);
    vb = mx_mfma<1>(ap[h], mx_b(r.vc[5][h]), vb, sp);
    va = mx_mfma<2>(ap[h], mx_b(r.vc[2][h]), va, sp);
    vb = mx_mfma<2>(ap[h], mx_b(r.vc[6][h]), vb, sp);
    va = mx_mfma<3>(ap[h], mx_b(r.vc[3][h]), va, sp);
    vb = mx_mfma<3>(ap[h], mx_b(r.vc[7][h]), vb, sp);
  }
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
template <int G>
struct alignas(16) WaveLds {
  uint8_t qa[4 * 128];                  // q' digit rows of the current page
  uint8_t pa[MxPage<G>::NB * 4 * 128];  // p' digit rows, one block per 128 slots
  float fin[4][D];                      // fp16-path fold, then this wave's accumulator
};

// G <= 128 fits 128 VGPRs (4 waves per SIMD); G = 256 holds twice the codes.
// kStep: a fused step's decode (the new token, counter advances, the store).
template <int G, bool kStep>
__global__ __launch_bounds__(256, G <= 128 ? 4 : 3) void decode_kernel(Arena a, const __half* __restrict__ q,
                                                     __half* __restrict__ out, int S,
                                                     HeadOrder order, StepArgs step) {
  __shared__ WaveLds<G> lds_all[kWaves];
  __shared__ float mg_m[kWaves], mg_l[kWaves];
  __shared__ uint32_t mg_last;
  // The prologue (head order, counters, query) is a chain of dependent loads:
  // at the top priority it is not held back by the waves of work-groups
  // already in their page loops (each page then sets the priority by the
  // work left).
  __builtin_amdgcn_s_setprio(3);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  WaveLds<G>& L = lds_all[wave];
  const int s = blockIdx.x % S;
  const int bh = order.n ? int(order.bh[blockIdx.x]) : int(blockIdx.x / S);  // = b * H + h
  const int b = bh / a.Hkv;
  // the query row is read before the counters, so the two reads wait together
  const float qscale = a.sm_scale * kLog2e;
  const __half* qrow = q + size_t(bh) * D;
  const uint4 q8 = reinterpret_cast<const uint4*>(qrow)[lane & 15];
  // the lane's two channels: those of logical k = 2 lane, 2 lane + 1
  const int c0 = mx_item(2 * lane);
  const float qs0 = __half2float(qrow[c0]) * qscale, qs1 = __half2float(qrow[c0 + 2]) * qscale;

  const HeadCtr hc = head_counters<kStep>(a, step, b, bh);
  const int r_cnt = hc.r_cnt, head = hc.head, nb = hc.nb;
  // a fused step's writer (the head's only or last split) stores the new row
  // at the end: load it now
  uint4 piece{};
  if constexpr (kStep)
    if (threadIdx.x >= D && threadIdx.x < D + 32) piece = step_row_piece(step, bh, threadIdx.x - D);
  const int pc = min(a.P, a.G * nb);
  const int n_new = kStep ? 1 : 0;  // a fused step's new token, after the window
  const Split sp = split_of(nb, pc + r_cnt + n_new, s, S);
  const int p1 = sp.p1, t1 = sp.t1;
  const int buf = nb & 1;
  const Fp16Src base_src{pool_k(a, buf, bh), pool_v(a, buf, bh), ring_k(a, bh), ring_v(a, bh), pc,
                         head, a.C};
  const auto src = [&] {
    if constexpr (kStep)
      return Fp16StepSrc{base_src, pc + r_cnt, step.k + size_t(bh) * D, step.v + size_t(bh) * D};
    else
      return base_src;
  }();
  const uint8_t* pages = page_ptr(a, bh, 0);
  const int64_t PB = a.page_bytes;
  WaveState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.vmin = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.acc[k] = 0.f;
  // fp16 chunks (memory-heavy) are spread between pages (compute-heavy),
  // staggered by wave, so the work-group always mixes the two. A split of
  // several holds a chunk or so: it goes to a wave with fewer pages.
  int chunk = S > 1 ? first_chunk(sp, wave) : sp.t0 + wave * kF16Chunk;
  auto next_chunk = [&]() {
    Fp16State fs;
    fs.m = -INFINITY;
    fs.l = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) fs.acc[k] = 0.f;
    fp16_chunk(src, chunk, min(kF16Chunk, t1 - chunk), q8, qscale, fs, lane);
    chunk += kWaves * kF16Chunk;
    // fold (m, l, acc) of the chunk into the page state; acc changes layout
    // through LDS (channel 8*(lane&15)+e, row lane>>4 -> the lane's channels
    // 16(lane>>4) + (lane&15) and that + 64)
    const float M = fmaxf(st.m, fs.m);
    rescale_q(st, M);
    const float af = (fs.m == -INFINITY) ? 0.f : exp2_fast(fs.m - M);
    st.l = fmaf(fs.l, af, st.l);
    float4* f = reinterpret_cast<float4*>(&L.fin[lane >> 4][8 * (lane & 15)]);
    f[0] = make_float4(fs.acc[0] * af, fs.acc[1] * af, fs.acc[2] * af, fs.acc[3] * af);
    f[1] = make_float4(fs.acc[4] * af, fs.acc[5] * af, fs.acc[6] * af, fs.acc[7] * af);
    wave_lds_sync();
    const int ca = 16 * (lane >> 4) + (lane & 15);
    st.acc[0] += (L.fin[0][ca] + L.fin[1][ca]) + (L.fin[2][ca] + L.fin[3][ca]);
    st.acc[4] += (L.fin[0][ca + 64] + L.fin[1][ca + 64]) + (L.fin[2][ca + 64] + L.fin[3][ca + 64]);
    wave_lds_sync();
  };
  // With one split every CU holds several heads' work-groups, dispatched one
  // after another. A short pause after the query loads and before the page
  // loads lets the work-groups dispatched last read their counters and query
  // before the page loads of the first ones fill the memory queues (without
  // it their counters arrived ~1.8 us late and they finished last; at 32
  // sequences x 32 heads of 3-4K tokens, 51.4 against 53.2 us per decode).
  if (S == 1) __builtin_amdgcn_s_sleep(8);
  int n = 0;
  for (int u = sp.p0 + wave; u < p1; u += kWaves, ++n) {
    prio_by_work_left((p1 - u + kWaves - 1) / kWaves);
    MxPage<G> pr;
    mx_load<G>(pr, pages + size_t(u) * PB, lane, c0);
    mx_page<G>(pr, page_nvalid(a.G, a.P, u), qs0, qs1, L.qa, L.pa, st, lane);
    if ((n & 3) == wave && chunk < t1) next_chunk();
  }
  while (chunk < t1) next_chunk();

  // this wave's state -> LDS in channel order
  const float l_tot = wave_sum(st.l);
  const float v_tot = wave_sum(st.vmin);
  {
    const int ca = 16 * (lane >> 4) + (lane & 15);
    L.fin[0][ca] = ((st.acc[0] + st.acc[1]) + (st.acc[2] + st.acc[3])) + v_tot;
    L.fin[0][ca + 64] = ((st.acc[4] + st.acc[5]) + (st.acc[6] + st.acc[7])) + v_tot;
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
      st_coherent(part + 2 + c, A);
      if (c == 0) {
        st_coherent(part, M);
        st_coherent(part + 1, Ls);
      }
    }
  } else if (kStep && S == 1 && threadIdx.x < D + 32) {
    // a fused step with one split: this work-group is the head's only reader
    // of its counters, so it stores the new token and the counters itself
    step_store(a, bh, hc, threadIdx.x - D, piece);
  }
  // several splits: the last one to finish merges them (every split has read
  // the head's counters and window by then, so it is also the step's writer)
  if (S > 1 && last_split(a, bh, S, &mg_last)) {
    if (threadIdx.x < D)
      out[size_t(bh) * D + threadIdx.x] =
          __float2half_rn(merge_partials<true>(partial_ptr(a, b, bh % a.Hq, 0), S, threadIdx.x));
    else if (kStep && threadIdx.x < D + 32)
      step_store(a, bh, hc, threadIdx.x - D, piece);
    if (threadIdx.x == 0) reset_ticket(a, bh);
  }
}

template <bool kStep>
hipError_t launch_g(const Arena& a, const __half* qh, __half* oh, int S, const HeadOrder& order,
                    const StepArgs& step, hipStream_t s) {
  const dim3 grid(unsigned(a.B) * a.Hkv * S);
  switch (a.G) {
    case 64: hipLaunchKernelGGL((decode_kernel<64, kStep>), grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order, step); break;
    case 128: hipLaunchKernelGGL((decode_kernel<128, kStep>), grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order, step); break;
    case 256: hipLaunchKernelGGL((decode_kernel<256, kStep>), grid, dim3(64 * kWaves), 0, s, a, qh, oh, S, order, step); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int decode_wgs_per_cu(const Arena& a) {
  if (a.Hq != a.Hkv) return decode_gqa_wgs_per_cu(a);
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (a.G) {
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<64, false>, 64 * kWaves, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<128, false>, 64 * kWaves, 0); break;
    case 256: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<256, false>, 64 * kWaves, 0); break;
    default: break;
  }
  return e == hipSuccess ? n : 0;
}

hipError_t launch_decode(const Arena& a, const void* q, void* out, int S, const HeadOrder& order,
                         const StepArgs& step, hipStream_t s) {
  const __half* qh = static_cast<const __half*>(q);
  __half* oh = static_cast<__half*>(out);
  hipError_t e;
  if (a.Hq != a.Hkv) {
    e = launch_decode_gqa(a, q, out, S, order, step, s);
  } else {
    e = step.k ? launch_g<true>(a, qh, oh, S, order, step, s)
               : launch_g<false>(a, qh, oh, S, order, step, s);
  }
  return e;
}

}  // namespace ott
