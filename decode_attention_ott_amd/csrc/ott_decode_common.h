// Device helpers shared by the decode kernels (gfx950, wave64): cross-lane
// reductions, streaming loads, the online-softmax rescale and the fp16-token
// (outlier pool + recent window) chunk walker.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ott_device.h"

namespace ott {
namespace dec {
using namespace dev;

constexpr int kWaves = 4;           // waves (work items) per work-group

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

// every lane of a 16-lane row receives the row's sum
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
}
// Row maxima compared as unsigned integers: a float's bits with the sign bit
// flipped (all bits when negative) order like the float (no NaN), and
// non-negative floats order like their bits. An unsigned maximum folds into
// its DPP move (0 is its identity), one instruction per step; a float maximum
// of a moved value first quiets its input, four instructions per step.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kQuadSwap1, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kQuadSwap2, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kHalfMirror, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kRowMirror, 0xF, 0xF, false)));
  return v;
}
// x >= 0 (or -0) in every lane
__device__ __forceinline__ float row_max_nonneg(float x) {
  return __uint_as_float(row_max_u32(__float_as_uint(x) & 0x7fffffffu));
}
// any x but NaN
__device__ __forceinline__ float row_max_ordered(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t u = row_max_u32(b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u));
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
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
// wave maxima through the same unsigned order (see row_max_u32)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max_u32(v);
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(uint32_t(r[0]), uint32_t(r[1]));
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ float wave_max_nonneg(float x) {
  return __uint_as_float(wave_max_u32(__float_as_uint(x) & 0x7fffffffu));
}
__device__ __forceinline__ float wave_max_ordered(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t u = wave_max_u32(b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u));
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
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
// x times the fp16 value in the high half of w: one mixed-precision FMA with a
// zero addend, the product rounded once as by a conversion and a multiply
// (only the sign of a zero product may differ).
__device__ __forceinline__ float mul_hi_f(float x, uint32_t w) {
  return __builtin_fmaf(x, hi_f(w), 0.0f);
}
__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// Issue priority from the pages a wave still has to process: the hardware
// favours older waves among equals, so without this the work-groups sharing a
// CU finish one after another and the CU runs its last stretch with few waves
// (little latency hiding). Waves with more work left go first instead, so the
// work-groups progress together. rem is wave-uniform.
__device__ __forceinline__ void prio_by_work_left(int rem) {
  if (rem >= 6) __builtin_amdgcn_s_setprio(3);
  else if (rem >= 4) __builtin_amdgcn_s_setprio(2);
  else if (rem >= 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// dword j (0..3) of a 16-byte vector
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

// Online softmax state (scores in log2 units) of one wave over fp16 tokens;
// a kernel folds it into its page state.
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

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  return x;
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

// The fp16 tokens of a fused step: token n_old (the last) is the step's new
// token, read from the step's input rows nk/nv.
struct Fp16StepSrc : Fp16Src {
  int n_old;  // pool + window tokens
  const __half* nk;
  const __half* nv;
  __device__ __forceinline__ const __half* k(int i) const { return i >= n_old ? nk : Fp16Src::k(i); }
  __device__ __forceinline__ const __half* v(int i) const { return i >= n_old ? nv : Fp16Src::v(i); }
};

// Counters of (sequence, KV head) bh as a step's decode sees them: a quantize
// step that becomes visible in this step advances the window and page count.
struct HeadCtr {
  int L, r_cnt, head, nb;
  bool adv;
};
__device__ __forceinline__ bool step_adv(const StepArgs& st, int b) {
  return st.k != nullptr && ((st.adv[b >> 5] >> (b & 31)) & 1u);
}
template <bool kStep>
__device__ __forceinline__ HeadCtr head_counters(const Arena& a, const StepArgs& st, int b, int bh) {
  const int32_t* ctr = counters(a, bh);
  if constexpr (!kStep) return HeadCtr{0, ctr[1], ctr[2], ctr[3], false};
  HeadCtr c{ctr[0], ctr[1], ctr[2], ctr[3], step_adv(st, b)};
  if (c.adv) {
    c.r_cnt -= a.G;
    c.head += a.G;
    if (c.head >= a.C) c.head -= a.C;
    c.nb += 1;
  }
  return c;
}

// Lane t (0..31) of the head's single writer: its 16-byte piece of the
// step's new K (t < 16) or V row of bh.
__device__ __forceinline__ uint4 step_row_piece(const StepArgs& st, int bh, int t) {
  return reinterpret_cast<const uint4*>((t < 16 ? st.k : st.v) + size_t(bh) * D)[t & 15];
}

// The step's new token of bh into window slot (head + r_cnt) % C, and the
// head's counters; called by lanes t = 0..31 of the head's single writer,
// each with its piece of the row (step_row_piece). The window head and page
// count are written only when they changed, so a quantize step reading them
// elsewhere never races with this write.
__device__ __forceinline__ void step_store(const Arena& a, int bh, const HeadCtr& c, int t,
                                           const uint4& piece) {
  int slot = c.head + c.r_cnt;
  if (slot >= a.C) slot -= a.C;
  uint4* dst = reinterpret_cast<uint4*>((t < 16 ? ring_k(a, bh) : ring_v(a, bh)) + size_t(slot) * D);
  dst[t & 15] = piece;
  if (t == 0) {
    int32_t* ctr = counters(a, bh);
    ctr[0] = c.L + 1;
    ctr[1] = c.r_cnt + 1;
    if (c.adv) {
      ctr[2] = c.head;
      ctr[3] = c.nb;
    }
  }
}

constexpr int kF16Pass = 4;                 // 4 tokens per pass
constexpr int kF16Chunk = 4 * kF16Pass;     // tokens per chunk

// The K and V rows of one chunk as this lane holds them.
struct Fp16Rows {
  uint4 k[kF16Pass], v[kF16Pass];
};

template <typename Src>
__device__ __forceinline__ void fp16_load(const Src& src, int base, int cnt, Fp16Rows& r,
                                          int lane) {
  const int rw = lane >> 4, c8 = lane & 15;
  // rows past the chunk read the chunk's last token (in bounds); their
  // weights are forced to zero. K and V rows are requested together.
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) r.k[p] = ld_nt4(src.k(base + min(4 * p + rw, cnt - 1)) + 8 * c8);
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) r.v[p] = ld_nt4(src.v(base + min(4 * p + rw, cnt - 1)) + 8 * c8);
}

// One query against a loaded chunk of cnt tokens, folded into st.
__device__ __forceinline__ void fp16_attend(const Fp16Rows& r, int cnt, const uint4& q8,
                                            float qscale, Fp16State& st, int lane) {
  const int rw = lane >> 4, c8 = lane & 15;
  float z[kF16Pass];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p) {
    float acc = fdot2(r.k[p].x, q8.x, 0.f);
    acc = fdot2(r.k[p].y, q8.y, acc);
    acc = fdot2(r.k[p].z, q8.z, acc);
    acc = fdot2(r.k[p].w, q8.w, acc);
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
    st.acc[0] = fmaf(w, lo_f(r.v[p].x), st.acc[0]);
    st.acc[1] = fmaf(w, hi_f(r.v[p].x), st.acc[1]);
    st.acc[2] = fmaf(w, lo_f(r.v[p].y), st.acc[2]);
    st.acc[3] = fmaf(w, hi_f(r.v[p].y), st.acc[3]);
    st.acc[4] = fmaf(w, lo_f(r.v[p].z), st.acc[4]);
    st.acc[5] = fmaf(w, hi_f(r.v[p].z), st.acc[5]);
    st.acc[6] = fmaf(w, lo_f(r.v[p].w), st.acc[6]);
    st.acc[7] = fmaf(w, hi_f(r.v[p].w), st.acc[7]);
  }
  if (c8 == 0) st.l += lsum;  // each row's tokens counted once
}

template <typename Src>
__device__ __forceinline__ void fp16_chunk(const Src& src, int base, int cnt, const uint4& q8,
                                           float qscale, Fp16State& st, int lane) {
  Fp16Rows r;
  fp16_load(src, base, cnt, r, lane);
  fp16_attend(r, cnt, q8, qscale, st, lane);
}

// Split s of S of one (sequence, KV head)'s cache: an even share of the pages
// [p0, p1) and an even share of the fp16 tokens [t0, t1) in whole chunks, so
// that every split holds about the same page bytes and at most a chunk or so
// of fp16 tokens (a chunk's load is one dependent wait whatever it holds, so
// neither one split with all of them nor every split with a sliver of one).
struct Split {
  int p0, p1, t0, t1;
};
__device__ __forceinline__ Split split_of(int nb, int n16, int s, int S) {
  const int nc = (n16 + kF16Chunk - 1) / kF16Chunk;
  return Split{s * nb / S, (s + 1) * nb / S, min(n16, kF16Chunk * (s * nc / S)),
               min(n16, kF16Chunk * ((s + 1) * nc / S))};
}
// First fp16 chunk of wave w in a split: chunks are dealt from the last wave
// down, since the last waves hold the fewest of the split's pages.
__device__ __forceinline__ int first_chunk(const Split& sp, int wave) {
  return sp.t0 + (kWaves - 1 - wave) * kF16Chunk;
}

// Partial state of split s for (sequence b, query head qh): {m, l, acc[D]}.
__device__ __forceinline__ float* partial_ptr(const Arena& a, int b, int qh, int s) {
  return reinterpret_cast<float*>(a.base + a.off_partials) +
         ((size_t(b) * a.Hq + qh) * a.max_splits + s) * (2 + D);
}

// Split-K partial states cross the XCDs: their L2 caches are not coherent
// with each other for plain accesses, so the partials are written and read
// with device-coherent (agent-scope) accesses, which reach the memory side
// (the compiler's release and acquire fences would instead write back and drop
// whole L2 contents at every split).
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K arrival, called by every thread of a work-group once its partial
// states are written (st_coherent): true, in every thread, for the head's
// last split to arrive, which then merges all S (ld_coherent). Each wave first
// waits for its own partial stores to complete, so every split's partials are
// in place before its ticket is taken. flag is LDS.
__device__ __forceinline__ bool last_split(const Arena& a, int bh, int S, uint32_t* flag) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): loads and stores of this wave
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = (__hip_atomic_fetch_add(ticket(a, bh), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             uint32_t(S - 1)) ? 1u : 0u;
  __syncthreads();
  return *flag != 0u;
}

// Channels c[n] of the merged outputs of N sets of S partial states
// {m, l, acc[D]} (log2 units), set n stored at part[n] + s * (2 + D): the
// partials are read 16 splits at a time with every load of all N sets in
// flight, then merged online,
// (M, L, A) <- (M', L e^(M-M') + sum l e^(m-M'), A e^(M-M') + sum acc e^(m-M')).
template <bool kCoherent, int N>
__device__ __forceinline__ void merge_partials_n(const float* const (&part)[N], int S,
                                                 const int (&c)[N], float (&out)[N]) {
  auto ld = [](const float* p) { return kCoherent ? ld_coherent(p) : *p; };
  constexpr int kChunk = 16;
  float M[N], Ls[N], A[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    M[n] = -INFINITY;
    Ls[n] = 0.f;
    A[n] = 0.f;
  }
  for (int i0 = 0; i0 < S; i0 += kChunk) {
    float m[N][kChunk], l[N][kChunk], v[N][kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k)
#pragma unroll
      for (int n = 0; n < N; ++n) {
        m[n][k] = -INFINITY;
        l[n][k] = 0.f;
        v[n][k] = 0.f;
        if (i0 + k < S) {  // uniform
          const float* p = part[n] + size_t(i0 + k) * (2 + D);
          m[n][k] = ld(p);
          l[n][k] = ld(p + 1);
          v[n][k] = ld(p + 2 + c[n]);
        }
      }
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float Mc = M[n];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) Mc = fmaxf(Mc, m[n][k]);
      if (Mc == -INFINITY) continue;
      const float f0 = (M[n] == -INFINITY) ? 0.f : exp2f(M[n] - Mc);
      Ls[n] *= f0;
      A[n] *= f0;
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const float f = (m[n][k] == -INFINITY) ? 0.f : exp2f(m[n][k] - Mc);
        Ls[n] = fmaf(l[n][k], f, Ls[n]);
        A[n] = fmaf(v[n][k], f, A[n]);
      }
      M[n] = Mc;
    }
  }
#pragma unroll
  for (int n = 0; n < N; ++n) out[n] = A[n] / Ls[n];
}

// Channel c of the merged output of the S partial states at part.
template <bool kCoherent = false>
__device__ __forceinline__ float merge_partials(const float* part, int S, int c) {
  const float* const ps[1] = {part};
  const int cs[1] = {c};
  float o[1];
  merge_partials_n<kCoherent, 1>(ps, S, cs, o);
  return o[0];
}

}  // namespace dec
}  // namespace ott
