// Cache-update kernels of the OTT path for gfx950 (CDNA4, wave64).
//
// Method: "Accurate KV Cache Quantization with Outlier Tokens Tracing"
// (arXiv 2505.10938); [Blog] = zijie-tian.site summary page, [Abs] =
// sciencestack.ai page (abstract and figure captions).
//
//   append_kernel    fp16 window update ([Blog] 3.3, residual window)
//   quantize_kernel  quantization stage: Key norms, pool competition, 2-bit
//                    pages ([Blog] 3.1, 3.2, flowchart; [Abs] Fig. 2 bottom)
//   prefill_top_kernel, prefill_select_kernel, prefill_pack_kernel  a whole
//                    prompt through the same steps: each segment's smallest P,
//                    the pool walk per segment, then every page at once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "ott_device.h"

namespace ott {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(Arena a, const uint4* __restrict__ k,
                                                     const uint4* __restrict__ v,
                                                     AppendCounts cnt) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int bh = b * a.Hkv + h;
  const int n = cnt.uniform >= 0 ? cnt.uniform : int(cnt.n[b]);
  if (cnt.init && threadIdx.x == 0) {  // first launch on the handle: counters from scratch
    int32_t* ctr = counters(a, bh);
    ctr[0] = n;
    ctr[1] = n;
    ctr[2] = 0;
    ctr[3] = 0;
    reset_ticket(a, bh);
  }
  if (n == 0) return;
  uint4* rk = reinterpret_cast<uint4*>(ring_k(a, bh));
  uint4* rv = reinterpret_cast<uint4*>(ring_v(a, bh));
  const size_t src = size_t(bh) * cnt.max_new * (D / 8);
  const int slot0 = cnt.slot0[b];
  for (int i = threadIdx.x; i < n * (D / 8); i += blockDim.x) {
    const int t = i / (D / 8), c = i % (D / 8);
    int slot = slot0 + t;
    slot -= (slot / a.C) * a.C;
    rk[size_t(slot) * (D / 8) + c] = k[src + i];
    rv[size_t(slot) * (D / 8) + c] = v[src + i];
  }
  if (!cnt.init && threadIdx.x == 0) {  // the only thread touching this head's counters here
    int32_t* ctr = counters(a, bh);
    ctr[0] += n;
    ctr[1] += n;
  }
}

// ---------------------------------------------------------------------------
// quantize: one work-group (1024 threads) per (sequence, KV head) with a full
// window; the host launches only the sequences that are due
// ---------------------------------------------------------------------------

// 2-bit code of x against (min m, scale s): clamp(rint(y), 0, 3) with
// y = fl32(fl32(x - m) / s), rint rounding half to even, computed without a
// division. The code counts the rounding thresholds y passes: y > 0.5,
// y >= 1.5, y > 2.5. With d = fl32(x - m) and q = d / s exact:
//   fl32(q) > 0.5  <=>  q > 0.5 + 2^-25  (the midpoint to the next float rounds
//                                        to the even 0.5)
//   fl32(q) >= 1.5 <=>  q >= 1.5 - 2^-24 (the midpoint below rounds up to 1.5)
//   fl32(q) > 2.5  <=>  q > 2.5 + 2^-23  (the midpoint above rounds down)
// For an fp16 scale, 0.5 s, 1.5 s and 2.5 s are exact in fp32, and no fp32 d
// lies strictly between c s and c s (1 +- 2^-24) (the float spacing there is
// wider), so the tests are d > 0.5 s, d >= 1.5 s, d > 2.5 s in fp32. A zero
// scale gives code 0 (thresholds +inf).
struct CodeThr {
  float m, t1, t2, t3;
};

__device__ __forceinline__ CodeThr code_thresholds(float m, float s) {
  if (!(s > 0.0f)) return CodeThr{m, INFINITY, INFINITY, INFINITY};
  return CodeThr{m, 0.5f * s, 1.5f * s, 2.5f * s};
}

// fp16 bits of a stored min or scale: a zero is stored as +0 whichever zero
// the reduction kept (the set may hold both; they compare equal, so fminf and
// fmaxf may return either).
__device__ __forceinline__ uint32_t meta_bits(float x) {
  const uint32_t h = __half_as_ushort(__float2half_rn(x));
  return h == 0x8000u ? 0u : h;
}

__device__ __forceinline__ uint32_t qcode(float x, const CodeThr& q) {
  const float d = __fsub_rn(x, q.m);
  return uint32_t(d > q.t1) + uint32_t(d >= q.t2) + uint32_t(d > q.t3);
}

// The pool's ranking key of a candidate (keys ascend, ties to the lower
// position): the squared Key norm (the method's rule), its negation, or a
// random fraction per position from the SplitMix64 generator.
__device__ __forceinline__ double retention_key(double n2, int pos, int rule) {
  if (rule == 1) return -n2;
  if (rule == 2) {
    uint64_t z = uint64_t(pos) + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return double(z >> 11) * 0x1p-53;
  }
  return n2;
}

constexpr int kStageRows = 128;  // member rows staged in LDS at a time (32 KiB)
constexpr int kQuantThreads = 1024;  // 16 waves: 4 per SIMD of the CU
constexpr int kMinMaxParts = kQuantThreads / D;  // partial K min/max per channel

struct QuantLds {
  __half* stage;  // [kStageRows][D]
  CodeThr* kq;    // [D] per channel c at (c % 16) * 8 + c / 16: K min and code thresholds
  CodeThr* vq;    // [G] per member: V min and code thresholds
  float* klo;     // [kMinMaxParts][D] partial K minima
  float* khi;     // [kMinMaxParts][D] partial K maxima
  double* n2;
  int* pos;
  int* src;
  int* rank;
  int* idx;       // member index of a candidate (counting)
  int* mem;
  int* wsum;      // [16] per-wave member counts of the group
};

// Dynamic LDS bytes of the QuantLds layout for (G, P) with a stage of
// `stage` rows (kStageRows, or 0 when the rows live in LDS whole).
__host__ __device__ inline size_t quant_lds_bytes(int G, int P, int stage = kStageRows) {
  const size_t nc = size_t(P) + G;
  return size_t(stage) * D * 2 + (D + size_t(G)) * sizeof(CodeThr) +
         2 * size_t(kMinMaxParts) * D * sizeof(float) + nc * sizeof(double) + 4 * nc * sizeof(int) +
         G * sizeof(int) + 16 * sizeof(int);
}

// LDS bytes of a quantize step that holds every candidate's K and V rows in
// LDS ([P + G][D] each, after the QuantLds layout without a stage).
__host__ __device__ inline size_t resident_lds_bytes(int G, int P) {
  return ((quant_lds_bytes(G, P, 0) + 15) & ~size_t(15)) + 2 * (size_t(P) + G) * D * sizeof(__half);
}

__device__ __forceinline__ QuantLds quant_lds(uint8_t* base, int NCmax, int G,
                                              int stage = kStageRows) {
  QuantLds q;
  q.stage = reinterpret_cast<__half*>(base);
  q.kq = reinterpret_cast<CodeThr*>(base + stage * D * sizeof(__half));
  q.vq = q.kq + D;
  q.klo = reinterpret_cast<float*>(q.vq + G);
  q.khi = q.klo + kMinMaxParts * D;
  q.n2 = reinterpret_cast<double*>(q.khi + kMinMaxParts * D);
  q.pos = reinterpret_cast<int*>(q.n2 + NCmax);
  q.src = q.pos + NCmax;
  q.rank = q.src + NCmax;
  q.idx = q.rank + NCmax;
  q.mem = q.idx + NCmax;
  q.wsum = q.mem + G;
  return q;
}

// Where pack_page finds the members' rows. Staged: rows are read from global
// memory through row functors (krow/vrow of a candidate's s.src) into the LDS
// stage, kStageRows members at a time. Resident: every candidate's rows are
// already in LDS, row i = candidate i (member t is candidate s.mem[t]).
template <typename KRow, typename VRow>
struct StagedRows {
  static constexpr bool kResident = false;
  KRow krow;
  VRow vrow;
};
struct ResidentRows {
  static constexpr bool kResident = true;
  const __half* k;  // [candidates][D]
  const __half* v;
};

// Copies rows [t0, t0+cnt) of the member list into the LDS stage with
// independent 16-byte loads (one round trip for the whole chunk).
template <typename RowFn>
__device__ __forceinline__ void stage_rows(const QuantLds& s, int t0, int cnt, RowFn row) {
  uint4* st = reinterpret_cast<uint4*>(s.stage);
  for (int i = threadIdx.x; i < cnt * (D / 8); i += blockDim.x) {
    const int t = i / (D / 8), c8 = i % (D / 8);
    st[i] = reinterpret_cast<const uint4*>(row(s.src[s.mem[t0 + t]]))[c8];
  }
}

// Squared Key norm of one fp16 row: fp64, summed in channel order 0..D-1.
__device__ __forceinline__ double sq_norm_fp64(const __half* __restrict__ k_row) {
  const uint4* row = reinterpret_cast<const uint4*>(k_row);
  uint4 w[D / 8];
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) w[c8] = row[c8];
  double acc = 0.0;
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) {
    const uint32_t ws[4] = {w[c8].x, w[c8].y, w[c8].z, w[c8].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double lo = double(__half2float(__ushort_as_half(uint16_t(ws[e] & 0xffffu))));
      const double hi = double(__half2float(__ushort_as_half(uint16_t(ws[e] >> 16))));
      acc = acc + lo * lo;
      acc = acc + hi * hi;
    }
  }
  return acc;
}

// Steps 1-3 of a quantize step for page nb: candidates (the pool's keys and
// positions from pkey/ppos, then the group's G tokens, rows (g_head + j) %
// g_mod of gk), their retention keys, ranks and the members in position order,
// all in LDS (s). The caller finishes the step. pre_n2, when given, holds the
// group tokens' squared norms (sq_norm_fp64 of their rows), computed earlier.
__device__ __forceinline__ void select_step(const Arena& a, int nb, const double* pkey,
                                            const int32_t* ppos, const __half* __restrict__ gk,
                                            int g_head, int g_mod, const QuantLds& s,
                                            const double* __restrict__ pre_n2 = nullptr) {
  const int G = a.G, P = a.P;
  const int tid = threadIdx.x;
  const int pc = min(P, G * nb);  // pool tokens before this step
  const int NC = pc + G;          // candidates: pool + group
  const int npc = min(P, NC);     // pool tokens after this step

  // 1. candidates; squared Key norms of the group, fp64 in channel order;
  //    their rank and member-index counters start at 0
  for (int i = tid; i < NC; i += blockDim.x) {
    s.rank[i] = 0;
    s.idx[i] = 0;
    if (i < pc) {
      s.n2[i] = pkey[i];
      s.pos[i] = ppos[i];
      s.src[i] = i;
    } else {
      const int j = i - pc;
      const int slot = (g_head + j) % g_mod;
      const double acc = pre_n2 ? pre_n2[j] : sq_norm_fp64(gk + size_t(slot) * D);
      s.n2[i] = retention_key(acc, G * nb + j, a.retention);
      s.pos[i] = G * nb + j;
      s.src[i] = slot | kRingFlag;
    }
  }
  __syncthreads();

  // 2. rank under (key, position). The pool's entries (i < pc) are in
  //    ascending (key, position) order and every pool position precedes every
  //    group position, so a pool entry's rank is its index plus the group keys
  //    below its key, and a group token's rank is the pool keys at or below its
  //    key (a binary search) plus the group tokens below it. Once the pool is
  //    full, a group token whose key is not below the pool's largest key ranks
  //    after all P pool entries: it is a member whatever its exact rank (set to
  //    NC), and neither it nor its comparisons change any other rank. So only
  //    the group tokens below that key (list `cl`, usually a few once the
  //    prompt is long) are counted, each against the others of the list. The
  //    comparisons are split over `parts` threads per candidate (branch-free,
  //    so the LDS reads pipeline) and summed with LDS atomics.
  const bool full = pc == P;
  int nC = G;  // group tokens that can enter the pool
  if (full) {
    const double kmax = P > 0 ? s.n2[pc - 1] : -INFINITY;
    const bool in_c = tid < G && s.n2[pc + tid] < kmax;
    if (tid < G && !in_c) s.rank[pc + tid] = NC;
    const uint64_t ball = __ballot(in_c);
    const int lane = tid & 63, wv = tid >> 6;
    if (lane == 0 && tid < G) s.wsum[wv] = __popcll(ball);
    __syncthreads();
    int before = 0;
    nC = 0;
    for (int w = 0; w < (G + 63) / 64; ++w) {
      nC += s.wsum[w];
      if (w < wv) before += s.wsum[w];
    }
    if (in_c)
      s.mem[before + __builtin_amdgcn_mbcnt_hi(uint32_t(ball >> 32),
                                               __builtin_amdgcn_mbcnt_lo(uint32_t(ball), 0))] =
          pc + tid;
    __syncthreads();
  }
  // candidate k of the list: pool entries first, then the group tokens that
  // can enter (in group order)
  const int M = pc + nC;
  auto cand = [&](int k) { return k < pc ? k : (full ? s.mem[k - pc] : k); };
  const int parts = M > 0 ? max(1, int(blockDim.x) / M) : 1;
  const int span = (nC + parts - 1) / parts;
  for (int x = tid; x < M * parts; x += blockDim.x) {
    const int e = x % M, part = x / M;
    const int i = cand(e);
    const int k0 = pc + part * span, k1 = min(M, k0 + span);
    const double ni = s.n2[i];
    const int pi = s.pos[i];
    int r = 0;
    if (i < pc) {
#pragma unroll 4
      for (int k = k0; k < k1; ++k) r += int(s.n2[cand(k)] < ni);
      if (part == 0) r += i;
    } else {
#pragma unroll 4
      for (int k = k0; k < k1; ++k) {
        const int jj = cand(k);
        const double nj = s.n2[jj];
        const int pj = s.pos[jj];
        r += int(nj < ni) | (int(nj == ni) & int(pj < pi));
      }
      if (part == 0) {  // pool keys <= ni
        int lo = 0, hi = pc;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s.n2[mid] <= ni) lo = mid + 1; else hi = mid;
        }
        r += lo;
      }
    }
    if (r) atomicAdd(&s.rank[i], r);
  }
  __syncthreads();

  // 3. members (rank >= npc) in position order: the evicted pool entries come
  //    first (their positions precede the group's), ordered by position among
  //    themselves; the group's members follow in group order (a prefix count
  //    of the member flags, by wave ballots)
  {
    const int pparts = pc > 0 ? max(1, int(blockDim.x) / pc) : 1;
    const int pspan = pc > 0 ? (pc + pparts - 1) / pparts : 0;
    for (int x = tid; x < pc * pparts; x += blockDim.x) {
      const int i = x % pc, j0 = (x / pc) * pspan, j1 = min(pc, j0 + pspan);
      if (s.rank[i] >= npc) {
        const int pi = s.pos[i];
        int c = 0;
#pragma unroll 4
        for (int j = j0; j < j1; ++j) c += int(s.rank[j] >= npc) & int(s.pos[j] < pi);
        if (c) atomicAdd(&s.idx[i], c);
      }
    }
    // group token g = tid (< G <= 256: the first G / 64 waves)
    const bool in_group = tid < G;
    const bool mflag = in_group && s.rank[pc + tid] >= npc;
    const uint64_t ball = __ballot(mflag);
    const int lane = tid & 63, wv = tid >> 6;
    const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(ball >> 32),
                                                __builtin_amdgcn_mbcnt_lo(uint32_t(ball), 0));
    if (lane == 0 && tid < G) s.wsum[wv] = __popcll(ball);
    __syncthreads();
    if (mflag) {
      int before = 0, total = 0;
      for (int w = 0; w < (G + 63) / 64; ++w) {
        total += s.wsum[w];
        if (w < wv) before += s.wsum[w];
      }
      const int n_evicted = (NC - npc) - total;
      s.idx[pc + tid] = n_evicted + before + below;
    }
  }
  __syncthreads();
  for (int i = tid; i < NC; i += blockDim.x)
    if (s.rank[i] >= npc) s.mem[s.idx[i]] = i;
  __syncthreads();
}

// Steps 4-6 of a quantize step: the page pg from its n_valid members (s.mem
// in position order, rows krow(s.src[m]) and vrow(s.src[m])): Key (min, scale)
// per channel and codes, Value (min, scale) per member and codes, zero padding.
template <typename Rows>
__device__ __forceinline__ void pack_page(const Arena& a, uint8_t* pg, const QuantLds& s,
                                          int n_valid, const Rows& rows) {
  const int G = a.G;
  const int tid = threadIdx.x;
  // member rows: chunks of the stage, or one chunk of all members in LDS
  constexpr bool kRes = Rows::kResident;
  const int chunk_rows = kRes ? max(n_valid, 1) : kStageRows;
  const int n_chunks = (n_valid + chunk_rows - 1) / chunk_rows;
  // row of member t0 + t (t within the chunk starting at t0)
  auto krow_of = [&](int t0, int t) -> const __half* {
    if constexpr (kRes) return rows.k + size_t(s.mem[t0 + t]) * D;
    else return s.stage + size_t(t) * D;
  };
  auto vrow_of = [&](int t0, int t) -> const __half* {
    if constexpr (kRes) return rows.v + size_t(s.mem[t0 + t]) * D;
    else return s.stage + size_t(t) * D;
  };
  // 4. Key (min, scale) per channel over the members: kMinMaxParts partial
  //    scans per channel, then one thread per channel combines them
  {
    float lo = INFINITY, hi = -INFINITY;
    const int c = tid % D, part = tid / D;  // blockDim.x == kMinMaxParts * D
    for (int ch = 0; ch < n_chunks; ++ch) {
      const int t0 = ch * chunk_rows, cnt = min(chunk_rows, n_valid - t0);
      if constexpr (!kRes) {
        stage_rows(s, t0, cnt, rows.krow);
        __syncthreads();
      }
#pragma unroll 4
      for (int t = part; t < cnt; t += kMinMaxParts) {
        const float x = __half2float(krow_of(t0, t)[c]);
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
      if constexpr (!kRes) __syncthreads();
    }
    s.klo[part * D + c] = lo;
    s.khi[part * D + c] = hi;
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int p2 = 1; p2 < kMinMaxParts; ++p2) {
        lo = fminf(lo, s.klo[p2 * D + tid]);
        hi = fmaxf(hi, s.khi[p2 * D + tid]);
      }
      if (n_valid == 0) lo = hi = 0.f;
      const uint32_t lo_b = meta_bits(lo);
      const uint32_t sc_b = meta_bits(__fdiv_rn(__fsub_rn(hi, lo), 3.0f));
      s.kq[(tid % 16) * (D / 16) + tid / 16] =
          code_thresholds(__half2float(__ushort_as_half(uint16_t(lo_b))),
                          __half2float(__ushort_as_half(uint16_t(sc_b))));
      reinterpret_cast<uint32_t*>(pg + kmeta_off(G))[tid] = lo_b | (sc_b << 16);
    }
  }
  __syncthreads();
  // 5. K codes, token-major: dword (t, j) = channels 16j..16j+15 of member t
  uint32_t* kc = reinterpret_cast<uint32_t*>(pg + kcode_off(G));
  for (int ch = 0; ch < n_chunks; ++ch) {
    const int t0 = ch * chunk_rows, cnt = min(chunk_rows, n_valid - t0);
    if constexpr (!kRes) {
      if (n_chunks > 1) {  // a single chunk is still staged from step 4
        stage_rows(s, t0, cnt, rows.krow);
        __syncthreads();
      }
    }
    const int jk = tid % (D / 16);  // this thread's 16 channels: 16*jk .. 16*jk+15
    CodeThr kq[16];  // the 8 blocks a wave reads for one cc are 128 contiguous bytes
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) kq[cc] = s.kq[cc * (D / 16) + jk];
    for (int w = tid; w < cnt * (D / 16); w += blockDim.x) {
      const int t = w / (D / 16), j = jk;
      const uint4* row = reinterpret_cast<const uint4*>(krow_of(t0, t) + 16 * j);
      const uint4 r0 = row[0], r1 = row[1];
      const uint32_t hw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      uint32_t word = 0;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const uint16_t bits = uint16_t(cc & 1 ? hw[cc >> 1] >> 16 : hw[cc >> 1] & 0xffffu);
        word |= qcode(__half2float(__ushort_as_half(bits)), kq[cc]) << (2 * cc);
      }
      kc[(t0 + t) * (D / 16) + j] = word;
    }
    __syncthreads();
  }
  for (int w = n_valid * (D / 16) + tid; w < G * (D / 16); w += blockDim.x) kc[w] = 0u;

  // 6. Values: per member (min, scale) over its channels, then V codes,
  //    channel-major: dword (c, j) = slots 16j..16j+15 of channel c
  uint32_t* vc = reinterpret_cast<uint32_t*>(pg + vcode_off(G));
  uint32_t* vmeta = reinterpret_cast<uint32_t*>(pg + vmeta_off(G));
  const int vdw = G / 16;
  for (int ch = 0; ch < n_chunks; ++ch) {
    const int t0 = ch * chunk_rows, cnt = min(chunk_rows, n_valid - t0);
    if constexpr (!kRes) {
      stage_rows(s, t0, cnt, rows.vrow);
      __syncthreads();
    }
    {
      // 8 lanes per member, 16 channels each (rotated per member against bank
      // conflicts), combined with cross-lane swaps inside the 8; blockDim / 8
      // members per pass
      for (int tb = 0; tb < cnt; tb += int(blockDim.x) / 8) {
        const int t = tb + (tid >> 3), part = tid & 7;
        float mn = INFINITY, mx = -INFINITY;
        if (t < cnt) {
          const __half* row = vrow_of(t0, t);
#pragma unroll
          for (int i = 0; i < D / 8; ++i) {
            const float x = __half2float(row[(part * (D / 8) + i + 2 * t) % D]);
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
          }
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          mn = fminf(mn, __shfl_xor(mn, o));
          mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        if (t < cnt && part == 0) {
          const uint32_t mn_b = meta_bits(mn);
          const uint32_t sc_b = meta_bits(__fdiv_rn(__fsub_rn(mx, mn), 3.0f));
          s.vq[t0 + t] = code_thresholds(__half2float(__ushort_as_half(uint16_t(mn_b))),
                                         __half2float(__ushort_as_half(uint16_t(sc_b))));
          vmeta[t0 + t] = mn_b | (sc_b << 16);
        }
      }
    }
    __syncthreads();
    // dwords whose 16 slots start inside this chunk (chunks are multiples of 16)
    const int jw0 = t0 / 16, jw1 = (t0 + cnt + 15) / 16;
    for (int w = tid; w < D * (jw1 - jw0); w += blockDim.x) {
      const int c = w % D, j = jw0 + w / D;
      uint32_t word = 0;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const int t = 16 * j + cc;
        if (t < n_valid)
          word |= qcode(__half2float(vrow_of(t0, t - t0)[c]), s.vq[t]) << (2 * cc);
      }
      vc[c * vdw + j] = word;
    }
    __syncthreads();
  }
  for (int t = n_valid + tid; t < G; t += blockDim.x) vmeta[t] = 0u;
  {
    const int jfirst = (n_valid + 15) / 16;  // dwords holding no member
    for (int w = tid; w < D * (vdw - jfirst); w += blockDim.x)
      vc[(w / (vdw - jfirst)) * vdw + jfirst + w % (vdw - jfirst)] = 0u;
  }
}

// One quantize step of (sequence, KV head) bh: the group's G tokens are rows
// (g_head + j) % g_mod of gk/gv (the window ring, or a prompt), competing with
// the pool of buffer nb & 1; writes page nb, the new pool into the other
// buffer and the page's member list. Counters are the caller's.
// kResident: every candidate's K and V rows, and the pool's keys and
// positions, are loaded into LDS first, all in one round trip, and every later
// phase reads them there (resident_lds_bytes of LDS); otherwise the members'
// rows are staged from global memory for the Key and the Value halves.
template <bool kResident>
__device__ __forceinline__ void quantize_step(const Arena& a, int bh, int nb,
                                              const __half* __restrict__ gk,
                                              const __half* __restrict__ gv, int g_head,
                                              int g_mod, uint8_t* lds_raw) {
  const int G = a.G, P = a.P;
  const int tid = threadIdx.x;
  const int pc = min(P, G * nb);
  const int NC = pc + G;
  const int npc = min(P, NC);
  const int n_valid = NC - npc;
  const int cur = nb & 1, nxt = cur ^ 1;
  QuantLds s = quant_lds(lds_raw, P + G, G, kResident ? 0 : kStageRows);

  const __half* pk = pool_k(a, cur, bh);
  const __half* pv = pool_v(a, cur, bh);
  auto krow = [&](int src) -> const __half* {
    return (src & kRingFlag) ? gk + size_t(src & ~kRingFlag) * D : pk + size_t(src) * D;
  };
  auto vrow = [&](int src) -> const __half* {
    return (src & kRingFlag) ? gv + size_t(src & ~kRingFlag) * D : pv + size_t(src) * D;
  };
  __half* kr = reinterpret_cast<__half*>(lds_raw + ((quant_lds_bytes(G, P, 0) + 15) & ~size_t(15)));
  __half* vr = kr + size_t(P + G) * D;
  if constexpr (kResident) {
    // 0. candidate i's rows into LDS row i (pool entries, then the group), the
    //    pool's keys and positions into the candidate arrays
    const double* pkey = pool_n2(a, cur, bh);
    const int32_t* ppos = pool_pos(a, cur, bh);
    for (int x = tid; x < NC * (D / 8); x += blockDim.x) {
      const int i = x / (D / 8), c8 = x % (D / 8);
      const int row = i < pc ? i : (g_head + i - pc) % g_mod;
      const __half* ks = (i < pc ? pk : gk) + size_t(row) * D;
      const __half* vs = (i < pc ? pv : gv) + size_t(row) * D;
      reinterpret_cast<uint4*>(kr + size_t(i) * D)[c8] = reinterpret_cast<const uint4*>(ks)[c8];
      reinterpret_cast<uint4*>(vr + size_t(i) * D)[c8] = reinterpret_cast<const uint4*>(vs)[c8];
    }
    for (int i = tid; i < pc; i += blockDim.x) {
      s.n2[i] = pkey[i];
      s.pos[i] = ppos[i];
    }
    __syncthreads();
    // 1-3 with the group's rows at LDS rows pc..pc+G-1
    select_step(a, nb, s.n2, s.pos, kr + size_t(pc) * D, 0, G, s);
    pack_page(a, page_ptr(a, bh, nb), s, n_valid, ResidentRows{kr, vr});
  } else {
    select_step(a, nb, pool_n2(a, cur, bh), pool_pos(a, cur, bh), gk, g_head, g_mod, s);
    pack_page(a, page_ptr(a, bh, nb), s, n_valid,
              StagedRows<decltype(krow), decltype(vrow)>{krow, vrow});
  }
  // 8. the new pool, slot = rank, into the other buffer
  __half* nk = pool_k(a, nxt, bh);
  __half* nv = pool_v(a, nxt, bh);
  for (int w = tid; w < NC * (D / 8); w += blockDim.x) {
    const int i = w / (D / 8), c8 = w % (D / 8);
    const int r = s.rank[i];
    if (r < npc) {
      const __half* ks = kResident ? kr + size_t(i) * D : krow(s.src[i]);
      const __half* vs = kResident ? vr + size_t(i) * D : vrow(s.src[i]);
      reinterpret_cast<uint4*>(nk + size_t(r) * D)[c8] = reinterpret_cast<const uint4*>(ks)[c8];
      reinterpret_cast<uint4*>(nv + size_t(r) * D)[c8] = reinterpret_cast<const uint4*>(vs)[c8];
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
}

template <bool kResident>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(Arena a, QuantizeList due) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const int h = blockIdx.x, b = due.b[blockIdx.y];
  const int bh = b * a.Hkv + h;
  int32_t* ctr = counters(a, bh);
  if (due.deferred) {
    // a fused step: the host picked this sequence; the step's decode advances
    // the counters (it may be writing the window count and length meanwhile,
    // so only the window head and page count are read here)
    quantize_step<kResident>(a, bh, ctr[3], ring_k(a, bh), ring_v(a, bh), ctr[2], a.C, lds_raw);
    return;
  }
  const int r_cnt = ctr[1], head = ctr[2], nb = ctr[3];
  if (r_cnt < a.C) return;  // window not full: nothing to do for this sequence
  quantize_step<kResident>(a, bh, nb, ring_k(a, bh), ring_v(a, bh), head, a.C, lds_raw);
  if (threadIdx.x == 0) {
    ctr[1] = r_cnt - a.G;
    ctr[2] = (head + a.G) % a.C;
    ctr[3] = nb + 1;
  }
}

// ---------------------------------------------------------------------------
// prefill: a prompt of L_b tokens per sequence into an empty cache, with the
// same result as appending it and running every due quantize step in order.
// A window is full at R+G tokens and a step removes G, so the prompt makes
// nq = floor((L - R) / G) pages (0 when L < R + G).
// The pool after step n holds the P smallest (key, position) pairs of all the
// tokens of groups 0..n: a step keeps the P smallest of the pool and the group,
// and the P smallest of a union are among the P smallest of each of its parts.
// So the groups are cut into segments of `seg` groups, and a segment's walk
// can start from the merge of the earlier segments' own P smallest. Kernels,
// after prefill_norms_kernel:
//   prefill_top_kernel     one work-group per (segment, sequence, KV head):
//       the segment's P smallest pairs, ascending (a radix select on the key
//       bits, ties in position order), into the segment's page slots.
//   prefill_select_kernel  one work-group per (segment, sequence, KV head):
//       the start pool from the earlier segments' tops, then the walk over the
//       segment's groups in position order on keys alone (the pool's keys and
//       positions stay in LDS from step to step): each step's members go to
//       the page's member list; the last segment then writes the final pool
//       and the one before it (the two pool buffers single steps would leave),
//       the window and the counters.
//   prefill_pack_kernel    one work-group per page slice (the Key channels or
//       the Value members of a page, at most 32 KiB of rows): its bytes from
//       the members' rows, read from the prompt by position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int prefill_pages(const Arena& a, int L) {
  return L >= a.R + a.G ? (L - a.R) / a.G : 0;
}

// The squared Key norms of every group token of the prompt, all pages of all
// heads at once: page n's G norms go to the first 8 G bytes of page n's own
// slot, which prefill_pack_kernel overwrites with the page afterwards.
__device__ __forceinline__ double* prefill_norms(const Arena& a, int bh, int n) {
  return reinterpret_cast<double*>(page_ptr(a, bh, n));
}

// One work-group of G threads per page; wave w takes tokens 64 w .. 64 w + 63.
// The rows reach each lane through LDS: a wave loads 8 half-rows (128 bytes
// each) per instruction, stores them with rows padded to 9 pieces (against bank
// conflicts), and each lane then sums its own token's channels in order.
__global__ __launch_bounds__(256) void prefill_norms_kernel(Arena a, const __half* __restrict__ k,
                                                            int64_t max_len, PrefillLens lens) {
  extern __shared__ uint4 tile_raw[];  // per wave: 64 half-rows of 8 pieces, padded to 9
  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.Hkv + h;
  if (n >= prefill_pages(a, lens.len[b])) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint4* kb =
      reinterpret_cast<const uint4*>(k + (size_t(bh) * max_len + size_t(n) * a.G + 64 * wv) * D);
  uint4* t = tile_raw + wv * 64 * 9;
  double acc = 0.0;
  for (int hf = 0; hf < 2; ++hf) {
    uint4 x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = kb[(8 * r + lane / 8) * (D / 8) + 8 * hf + lane % 8];
#pragma unroll
    for (int r = 0; r < 8; ++r) t[(8 * r + lane / 8) * 9 + lane % 8] = x[r];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint4 w = t[lane * 9 + p];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double lo = double(__half2float(__ushort_as_half(uint16_t(ws[e] & 0xffffu))));
        const double hi = double(__half2float(__ushort_as_half(uint16_t(ws[e] >> 16))));
        acc = acc + lo * lo;
        acc = acc + hi * hi;
      }
    }
    __syncthreads();
  }
  prefill_norms(a, bh, n)[64 * wv + lane] = acc;
}

// Unsigned bits of a retention key that order as the key does: negative keys
// inverted, non-negative ones with the top bit set. Zeros come with one sign
// under every rule (a norm is +0, its negation -0, a random fraction +0), so
// equal keys have equal bits.
__device__ __forceinline__ uint64_t key_bits(double x) {
  const uint64_t u = uint64_t(__double_as_longlong(x));
  return (u >> 63) ? ~u : (u | (1ull << 63));
}
__device__ __forceinline__ double key_of_bits(uint64_t u) {
  return __longlong_as_double((long long)((u >> 63) ? (u & ~(1ull << 63)) : ~u));
}
__device__ __forceinline__ uint64_t shr64(uint64_t u, int n) { return n >= 64 ? 0 : u >> n; }

// A segment's smallest (key, position) pairs, ascending, sit in the free bytes
// of its own page slots (bytes [8 G, page_bytes) of each, rounded down to 8,
// after the slot's norms): P keys, then P positions. The pack overwrites them.
__device__ __forceinline__ uint8_t* seg_top_at(const Arena& a, int bh, int g0, size_t off) {
  const size_t f = (size_t(a.page_bytes) - 8 * size_t(a.G)) & ~size_t(7);
  return page_ptr(a, bh, g0 + int(off / f)) + 8 * size_t(a.G) + off % f;
}
__device__ __forceinline__ double* seg_top_key(const Arena& a, int bh, int g0, int i) {
  return reinterpret_cast<double*>(seg_top_at(a, bh, g0, 8 * size_t(i)));
}
__device__ __forceinline__ int32_t* seg_top_pos(const Arena& a, int bh, int g0, int i) {
  return reinterpret_cast<int32_t*>(seg_top_at(a, bh, g0, 8 * size_t(a.P) + 4 * size_t(i)));
}

// 512 threads with 16 keys each: two work-groups per CU (81 VGPRs); 1024
// threads took 59 against 38 us for the 24 segments of 40 heads at 128K
constexpr int kTopThreads = 512;
constexpr int kTopPerThread = 16;  // a segment holds at most 16 * 512 tokens
constexpr int kMaxPool = 512;

// The min(P, seg G) smallest (key, position) pairs of segment blockIdx.x's
// tokens, ascending. Radix select from the top bit that differs between the
// smallest and largest key, 8 bits a pass: a histogram of the next digit among
// the tokens still on the boundary picks the digit where the count reaches P.
// The pairs below the final boundary are all taken; on it, the first ones in
// position order. Then ranked by (key, position). The last segment of a
// sequence has no successor to read its pairs and is skipped.
__global__ __launch_bounds__(kTopThreads) void prefill_top_kernel(Arena a, PrefillLens lens,
                                                                    int seg) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t red[2][kTopThreads / 64];
  __shared__ int pick[3];  // digit, pairs below it, pairs on it
  __shared__ int wcnt[kTopThreads / 64];
  __shared__ int n_sel;
  __shared__ double sel_k[kMaxPool];
  __shared__ int32_t sel_p[kMaxPool];
  __shared__ int sel_r[kMaxPool];
  const int sg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.Hkv + h;
  const int nq = prefill_pages(a, lens.len[b]);
  const int g0 = sg * seg;
  if (g0 + seg >= nq) return;
  const int G = a.G, n = seg * G, take = min(a.P, n);
  if (take == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int kWavesT = kTopThreads / 64;

  uint64_t u[kTopPerThread];
  uint64_t mn = ~0ull, mx = 0;
#pragma unroll
  for (int k = 0; k < kTopPerThread; ++k) {
    const int j = tid + k * kTopThreads;
    u[k] = 0;
    if (j < n) {
      const double x = retention_key(prefill_norms(a, bh, g0 + j / G)[j % G], g0 * G + j,
                                     a.retention);
      u[k] = key_bits(x);
      mn = min(mn, u[k]);
      mx = max(mx, u[k]);
    }
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    red[0][wv] = mn;
    red[1][wv] = mx;
  }
  if (tid == 0) n_sel = 0;
  __syncthreads();
  mn = red[0][0];
  mx = red[1][0];
  for (int w = 1; w < kWavesT; ++w) {
    mn = min(mn, red[0][w]);
    mx = max(mx, red[1][w]);
  }
  // boundary: tokens whose bits above `lo` equal `pre` (`bin` of them);
  // `need` of them are still to be taken
  int need = take, bin = n, lo = 0;
  uint64_t pre = mn;
  if (mn != mx) {
    lo = 64 - __clzll((long long)(mn ^ mx));
    pre = shr64(mn, lo);
    while (lo > 0) {
      const int nlo = max(lo - 8, 0);
      const uint32_t mask = (1u << (lo - nlo)) - 1u;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kTopPerThread; ++k)
        if (tid + k * kTopThreads < n && shr64(u[k], lo) == pre)
          atomicAdd(&hist[uint32_t(u[k] >> nlo) & mask], 1u);
      __syncthreads();
      if (wv == 0) {
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = hist[4 * lane + i];
          sum += c[i];
        }
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        uint32_t below = incl - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (below < uint32_t(need) && uint32_t(need) <= below + c[i]) {
            pick[0] = 4 * lane + i;
            pick[1] = int(below);
            pick[2] = int(c[i]);
          }
          below += c[i];
        }
      }
      __syncthreads();
      pre = (pre << (lo - nlo)) | uint64_t(pick[0]);
      need -= pick[1];
      bin = pick[2];
      lo = nlo;
      if (bin == need) break;  // the whole boundary is taken
    }
  }
  // take the pairs below the boundary, and the first `need` on it
  const bool split = bin > need;  // only with lo == 0: equal keys, by position
  int tie_base = 0;
#pragma unroll
  for (int k = 0; k < kTopPerThread; ++k) {
    const int j = tid + k * kTopThreads;
    const bool valid = j < n;
    const uint64_t hb = shr64(u[k], lo);
    const bool tie = valid && hb == pre;
    bool taken = valid && hb < pre;
    if (split) {
      if (k * kTopThreads >= n) break;  // uniform
      const uint64_t ball = __ballot(tie);
      const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(ball >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(uint32_t(ball), 0));
      if (lane == 0) wcnt[wv] = __popcll(ball);
      __syncthreads();
      int before = 0, total = 0;
      for (int w = 0; w < kWavesT; ++w) {
        total += wcnt[w];
        if (w < wv) before += wcnt[w];
      }
      __syncthreads();
      taken = taken || (tie && tie_base + before + below < need);
      tie_base += total;
    } else {
      taken = taken || tie;
    }
    if (taken) {  // exactly `take` of them
      const int slot = atomicAdd(&n_sel, 1);
      if (slot < kMaxPool) {
        sel_k[slot] = key_of_bits(u[k]);
        sel_p[slot] = g0 * G + j;
      }
    }
  }
  for (int i = tid; i < take; i += blockDim.x) sel_r[i] = 0;
  __syncthreads();
  // ranks under (key, position), `parts` threads per pair
  const int parts = max(1, int(blockDim.x) / take);
  const int span = (take + parts - 1) / parts;
  for (int x = tid; x < take * parts; x += blockDim.x) {
    const int i = x % take, j0 = (x / take) * span, j1 = min(take, j0 + span);
    const double ki = sel_k[i];
    const int pi = sel_p[i];
    int r = 0;
#pragma unroll 4
    for (int j = j0; j < j1; ++j) {
      const double kj = sel_k[j];
      r += int(kj < ki) | (int(kj == ki) & int(sel_p[j] < pi));
    }
    if (r) atomicAdd(&sel_r[i], r);
  }
  __syncthreads();
  for (int i = tid; i < take; i += blockDim.x) {
    *seg_top_key(a, bh, g0, sel_r[i]) = sel_k[i];
    *seg_top_pos(a, bh, g0, sel_r[i]) = sel_p[i];
  }
}

// 512 threads, four work-groups per CU (8 waves per SIMD): the walk's steps
// are short phases between barriers, which the other work-groups fill.
constexpr int kWalkThreads = 512;
static_assert(kWalkThreads >= 256, "select_step gives each group token (G <= 256) a thread");
static_assert(kWalkThreads >= kMaxPool, "the start-pool merge gives each pair a thread");
__global__ __launch_bounds__(kWalkThreads) __attribute__((amdgpu_waves_per_eu(8)))
void prefill_select_kernel(
    Arena a, const __half* __restrict__ k, const __half* __restrict__ v, int64_t max_len,
    PrefillLens lens, int seg) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const int sg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.Hkv + h;
  const int L = lens.len[b];
  if (L == 0) {  // an empty sequence still gets its counters (the arena is not zeroed)
    if (sg == 0 && threadIdx.x == 0) {
      int32_t* ctr = counters(a, bh);
      ctr[0] = ctr[1] = ctr[2] = ctr[3] = 0;
      reset_ticket(a, bh);
    }
    return;
  }
  const int G = a.G, P = a.P, C = a.C;
  const int tid = threadIdx.x;
  const int nq = prefill_pages(a, L);
  const int g0 = sg * seg, g1 = min(nq, g0 + seg);
  if (sg > 0 && g0 >= nq) return;  // segment 0 runs even without pages: it writes the window
  const __half* kb = k + size_t(bh) * max_len * D;
  const __half* vb = v + size_t(bh) * max_len * D;
  QuantLds s = quant_lds(lds_raw, P + G, G, 0);
  // two pools of keys and positions after the QuantLds region
  double* pkey[2];
  int32_t* ppos[2];
  {
    uint8_t* base = lds_raw + ((quant_lds_bytes(G, P, 0) + 15) & ~size_t(15));
    pkey[0] = reinterpret_cast<double*>(base);
    pkey[1] = pkey[0] + P;
    ppos[0] = reinterpret_cast<int32_t*>(pkey[1] + P);
    ppos[1] = ppos[0] + P;
  }
  // the pool before step g0: the earlier segments' smallest pairs merged in
  // order, each merge keeping the P smallest of two ascending lists (a pair's
  // merged rank is its index plus the pairs of the other list below it); the
  // merges alternate buffers and end in buffer g0 & 1, which step g0 reads
  {
    int x = (g0 + sg) & 1, pc = 0;
    const int cb = min(P, seg * G);  // <= 512 = blockDim: one pair per thread
    // the next segment's pairs travel in registers while this merge runs
    double nk = 0.0;
    int np = 0;
    if (sg > 0 && tid < cb) {
      nk = *seg_top_key(a, bh, 0, tid);
      np = *seg_top_pos(a, bh, 0, tid);
    }
    for (int i = 0; i < sg; ++i) {
      if (tid < cb) {
        s.n2[tid] = nk;
        s.pos[tid] = np;
      }
      __syncthreads();
      if (i + 1 < sg && tid < cb) {
        nk = *seg_top_key(a, bh, (i + 1) * seg, tid);
        np = *seg_top_pos(a, bh, (i + 1) * seg, tid);
      }
      const int npc = min(P, pc + cb);
      for (int t = tid; t < pc + cb; t += blockDim.x) {
        const bool in_pool = t < pc;
        const int own = in_pool ? t : t - pc;
        const double kk = in_pool ? pkey[x][t] : s.n2[own];
        const int pp = in_pool ? ppos[x][t] : s.pos[own];
        const double* ok = in_pool ? s.n2 : pkey[x];
        const int32_t* op = in_pool ? s.pos : ppos[x];
        int lo = 0, hi = in_pool ? cb : pc;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (ok[mid] < kk || (ok[mid] == kk && op[mid] < pp)) lo = mid + 1; else hi = mid;
        }
        const int r = own + lo;
        if (r < npc) {
          pkey[x ^ 1][r] = kk;
          ppos[x ^ 1][r] = pp;
        }
      }
      __syncthreads();
      x ^= 1;
      pc = npc;
    }
  }
  int32_t* page_pos_all = reinterpret_cast<int32_t*>(a.base + a.off_page_pos);
  int32_t* page_nv_all = reinterpret_cast<int32_t*>(a.base + a.off_page_nvalid);
  for (int n = g0; n < g1; ++n) {
    const int pc = min(P, G * n), NC = pc + G, npc = min(P, NC), n_valid = NC - npc;
    const int cur = n & 1;
    select_step(a, n, pkey[cur], ppos[cur], kb + size_t(n) * G * D, 0, G, s,
                prefill_norms(a, bh, n));
    int32_t* pp = page_pos_all + (size_t(bh) * a.nb_max + n) * G;
    for (int t = tid; t < G; t += blockDim.x) pp[t] = t < n_valid ? s.pos[s.mem[t]] : -1;
    if (tid == 0) page_nv_all[size_t(bh) * a.nb_max + n] = n_valid;
    for (int i = tid; i < NC; i += blockDim.x) {
      const int r = s.rank[i];
      if (r < npc) {
        pkey[cur ^ 1][r] = s.n2[i];
        ppos[cur ^ 1][r] = s.pos[i];
      }
    }
    __syncthreads();
  }
  if (g1 < nq) return;  // a later segment finishes the sequence
  // pools: after nq steps in buffer nq & 1, after nq - 1 steps in the other one
  for (int back = 0; back < 2 && back < nq; ++back) {
    const int steps = nq - back, buf = steps & 1;
    const int cnt = min(P, G * steps);
    __half* dk = pool_k(a, buf, bh);
    __half* dv = pool_v(a, buf, bh);
    for (int w = tid; w < cnt * (D / 8); w += blockDim.x) {
      const int i = w / (D / 8), c8 = w % (D / 8);
      const int pos = ppos[buf][i];
      reinterpret_cast<uint4*>(dk + size_t(i) * D)[c8] =
          reinterpret_cast<const uint4*>(kb + size_t(pos) * D)[c8];
      reinterpret_cast<uint4*>(dv + size_t(i) * D)[c8] =
          reinterpret_cast<const uint4*>(vb + size_t(pos) * D)[c8];
      if (c8 == 0) {
        pool_pos(a, buf, bh)[i] = pos;
        pool_n2(a, buf, bh)[i] = pkey[buf][i];
      }
    }
  }
  // the window: the last L - G nq tokens, at the slots single steps would use
  const int rc = L - G * nq, head = (G * nq) % C;
  uint4* rk = reinterpret_cast<uint4*>(ring_k(a, bh));
  uint4* rv = reinterpret_cast<uint4*>(ring_v(a, bh));
  const uint4* sk = reinterpret_cast<const uint4*>(kb + size_t(G) * nq * D);
  const uint4* sv = reinterpret_cast<const uint4*>(vb + size_t(G) * nq * D);
  for (int i = tid; i < rc * (D / 8); i += blockDim.x) {
    const int t = i / (D / 8), c = i % (D / 8);
    const int slot = (head + t) % C;
    rk[size_t(slot) * (D / 8) + c] = sk[i];
    rv[size_t(slot) * (D / 8) + c] = sv[i];
  }
  if (tid == 0) {
    int32_t* ctr = counters(a, bh);
    ctr[0] = L;
    ctr[1] = rc;
    ctr[2] = head;
    ctr[3] = nq;
    reset_ticket(a, bh);
  }
}

constexpr int kPackThreads = 512;
constexpr int kPackRowBytes = 32768;  // member rows a pack work-group holds in LDS

// LDS of a prefill pack work-group: the rows of its slice, then the code
// thresholds (per channel or per member) and the partial Key minima and maxima.
__host__ __device__ inline size_t pack_lds_bytes() {
  return kPackRowBytes + 256 * sizeof(CodeThr) + 2 * kPackThreads * sizeof(float);
}

// Moves `pieces` 16-byte pieces of each of `cnt` rows into LDS (row i at
// rows + i * pieces * 16 bytes): piece tid % pieces of rows tid / pieces +
// (512 / pieces) r, the row indices first, then every load at once. Rows past
// `cnt` read row 0 of the prompt (present whenever a page is) and drop it.
template <typename RowOf>
__device__ __forceinline__ void pack_stage(uint4* rows, int pieces, int cnt, RowOf row_of,
                                           const __half* __restrict__ src, int piece0) {
  constexpr int kRounds = 4;  // cnt * pieces <= 4 * 512
  const int tid = threadIdx.x, pc = tid % pieces, t0 = tid / pieces, step = kPackThreads / pieces;
  int pos[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = t0 + r * step;
    pos[r] = t < cnt ? row_of(t) : 0;
  }
  uint4 x[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    x[r] = reinterpret_cast<const uint4*>(src + size_t(pos[r]) * D)[piece0 + pc];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = t0 + r * step;
    if (t < cnt) rows[t * pieces + pc] = x[r];
  }
}

// One slice of page n's bytes, from its members' rows read from the prompt by
// position, with the arithmetic of a single quantize step. A page is cut into
// 2 S slices of at most 32 KiB of rows (S = G / 128 at G = 256, else 1):
// q < S: the Key (min, scale) and codes of channels [q D / S, (q + 1) D / S)
// over all members; q >= S: the Value (min, scale) and codes of members
// [(q - S) G / S, (q - S + 1) G / S). blockIdx.x = 2 n + q at S = 1. At S = 2
// the slices of a page write the two halves of the same 128-byte lines (Key
// codes of a member, Value codes of a channel), so they run on one XCD (work-
// group i runs on XCD i mod 8, and the x dimension is padded to a multiple of
// 32), where the halves meet in its L2: blockIdx.x = 32 (n / 8) + 8 q + n % 8.
template <int S>
__global__ __launch_bounds__(kPackThreads) void prefill_pack_kernel(
    Arena a, const __half* __restrict__ k, const __half* __restrict__ v, int64_t max_len,
    PrefillLens lens) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const int xb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = S == 1 ? xb / 2 : (xb / 32) * 8 + xb % 8;
  const int q = S == 1 ? xb % 2 : (xb / 8) % 4;
  const int bh = b * a.Hkv + h;
  if (n >= prefill_pages(a, lens.len[b])) return;
  const int G = a.G, P = a.P, tid = threadIdx.x;
  const int pc = min(P, G * n);
  const int n_valid = pc + G - min(P, pc + G);
  __half* rows = reinterpret_cast<__half*>(lds_raw);
  CodeThr* thr = reinterpret_cast<CodeThr*>(lds_raw + kPackRowBytes);
  float* plo = reinterpret_cast<float*>(thr + 256);
  float* phi = plo + kPackThreads;
  const int32_t* pp = reinterpret_cast<const int32_t*>(a.base + a.off_page_pos) +
                      (size_t(bh) * a.nb_max + n) * G;
  uint8_t* pg = page_ptr(a, bh, n);
  auto member_pos = [&](int t) { return pp[t]; };
  if (q < S) {
    // Key slice: channels c0 .. c0 + DC - 1 of every member (row t at t * DC)
    constexpr int DC = D / S, kParts = kPackThreads / DC;
    const int c0 = q * DC;
    pack_stage(reinterpret_cast<uint4*>(rows), DC / 8, n_valid, member_pos,
               k + size_t(bh) * max_len * D, c0 / 8);
    __syncthreads();
    {
      const int c = tid % DC, part = tid / DC;
      float lo = INFINITY, hi = -INFINITY;
#pragma unroll 4
      for (int t = part; t < n_valid; t += kParts) {
        const float x = __half2float(rows[t * DC + c]);
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
      plo[tid] = lo;
      phi[tid] = hi;
    }
    __syncthreads();
    if (tid < DC) {
      float lo = plo[tid], hi = phi[tid];
#pragma unroll
      for (int p2 = 1; p2 < kParts; ++p2) {
        lo = fminf(lo, plo[p2 * DC + tid]);
        hi = fmaxf(hi, phi[p2 * DC + tid]);
      }
      if (n_valid == 0) lo = hi = 0.f;
      const int c = c0 + tid;
      const uint32_t lo_b = meta_bits(lo);
      const uint32_t sc_b = meta_bits(__fdiv_rn(__fsub_rn(hi, lo), 3.0f));
      thr[(c % 16) * (D / 16) + c / 16] =
          code_thresholds(__half2float(__ushort_as_half(uint16_t(lo_b))),
                          __half2float(__ushort_as_half(uint16_t(sc_b))));
      reinterpret_cast<uint32_t*>(pg + kmeta_off(G))[c] = lo_b | (sc_b << 16);
    }
    __syncthreads();
    // codes, token-major: dword (t, j) = channels 16 j .. 16 j + 15 of member
    // t (zero past the members); channel 16 j + cc's thresholds at cc * 8 + j.
    // The slice's dwords (t, j0 .. j0 + JS - 1) are gathered in LDS (over the
    // partial minima, no longer read) and stored 16 bytes at a time.
    uint32_t* kc = reinterpret_cast<uint32_t*>(pg + kcode_off(G));
    uint32_t* words = reinterpret_cast<uint32_t*>(plo);  // [G][JS]
    constexpr int JS = DC / 16;
    for (int w = tid; w < G * JS; w += kPackThreads) {
      const int t = w / JS, jj = w % JS, j = c0 / 16 + jj;
      uint32_t word = 0;
      if (t < n_valid) {
        const uint4* row = reinterpret_cast<const uint4*>(rows + t * DC + 16 * jj);
        const uint4 r0 = row[0], r1 = row[1];
        const uint32_t hw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
          const uint16_t bits = uint16_t(cc & 1 ? hw[cc >> 1] >> 16 : hw[cc >> 1] & 0xffffu);
          word |= qcode(__half2float(__ushort_as_half(bits)), thr[cc * (D / 16) + j]) << (2 * cc);
        }
      }
      words[w] = word;
    }
    __syncthreads();
    for (int w = tid; w < G * JS / 4; w += kPackThreads) {
      const int t = w / (JS / 4), u = w % (JS / 4);
      reinterpret_cast<uint4*>(kc + t * (D / 16) + c0 / 16)[u] =
          reinterpret_cast<const uint4*>(words)[w];
    }
    return;
  }
  // Value slice: members m0 .. m0 + MC - 1 (row t - m0 at (t - m0) * D)
  const int MC = G / S, m0 = (q - S) * MC;
  const int cnt = max(0, min(MC, n_valid - m0));
  pack_stage(reinterpret_cast<uint4*>(rows), D / 8, cnt, [&](int t) { return pp[m0 + t]; },
             v + size_t(bh) * max_len * D, 0);
  __syncthreads();
  // (min, scale) per member: 8 lanes per member, 8 channel pairs each (4-byte
  // reads, rotated per member against bank conflicts), combined by lane swaps
  uint32_t* vmeta = reinterpret_cast<uint32_t*>(pg + vmeta_off(G));
  const uint32_t* rows2 = reinterpret_cast<const uint32_t*>(rows);  // channel pairs
  for (int tb = 0; tb < MC; tb += kPackThreads / 8) {
    const int tl = tb + (tid >> 3), part = tid & 7, t = m0 + tl;
    float mn = INFINITY, mx = -INFINITY;
    if (tl < cnt) {
      const uint32_t* row = rows2 + tl * (D / 2);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const uint32_t w = row[(part * (D / 16) + i + tl) % (D / 2)];
        const float x0 = __half2float(__ushort_as_half(uint16_t(w & 0xffffu)));
        const float x1 = __half2float(__ushort_as_half(uint16_t(w >> 16)));
        mn = fminf(mn, fminf(x0, x1));
        mx = fmaxf(mx, fmaxf(x0, x1));
      }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (tl < MC && part == 0) {
      if (tl < cnt) {
        const uint32_t mn_b = meta_bits(mn);
        const uint32_t sc_b = meta_bits(__fdiv_rn(__fsub_rn(mx, mn), 3.0f));
        thr[tl] = code_thresholds(__half2float(__ushort_as_half(uint16_t(mn_b))),
                                  __half2float(__ushort_as_half(uint16_t(sc_b))));
        vmeta[t] = mn_b | (sc_b << 16);
      } else {
        vmeta[t] = 0u;
      }
    }
  }
  __syncthreads();
  // codes, channel-major: dword (c, j) = members 16 j .. 16 j + 15 of channel c
  // (zero past the members), a lane taking channels c and c + 1 (one 4-byte
  // read per member, one threshold read for both), gathered in LDS as [c][js]
  // and stored 16 bytes at a time
  uint32_t* vc = reinterpret_cast<uint32_t*>(pg + vcode_off(G));
  uint32_t* words = reinterpret_cast<uint32_t*>(plo);
  const int vdw = G / 16, js = MC / 16;
  for (int w = tid; w < (D / 2) * js; w += kPackThreads) {
    const int c2 = w % (D / 2), jj = w / (D / 2);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) {
      const int tl = 16 * jj + cc;
      if (tl < cnt) {
        const uint32_t x = rows2[tl * (D / 2) + c2];
        const CodeThr q = thr[tl];
        w0 |= qcode(__half2float(__ushort_as_half(uint16_t(x & 0xffffu))), q) << (2 * cc);
        w1 |= qcode(__half2float(__ushort_as_half(uint16_t(x >> 16))), q) << (2 * cc);
      }
    }
    words[(2 * c2) * js + jj] = w0;
    words[(2 * c2 + 1) * js + jj] = w1;
  }
  __syncthreads();
  for (int w = tid; w < D * js / 4; w += kPackThreads) {
    const int c = w / (js / 4), u = w % (js / 4);
    reinterpret_cast<uint4*>(vc + c * vdw + m0 / 16)[u] = reinterpret_cast<const uint4*>(words)[w];
  }
}

}  // namespace

hipError_t launch_append(const Arena& a, const void* k, const void* v, const AppendCounts& n,
                         hipStream_t s) {
  dim3 grid(a.Hkv, a.B);
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, s, a, static_cast<const uint4*>(k),
                     static_cast<const uint4*>(v), n);
  return hipGetLastError();
}

size_t quantize_lds_bytes(int G, int P) { return quant_lds_bytes(G, P); }

size_t prefill_select_lds_bytes(int G, int P) {
  return ((quant_lds_bytes(G, P, 0) + 15) & ~size_t(15)) + size_t(P) * 2 * (sizeof(double) + 4);
}

// Groups per prefill segment: segments enough for up to four walk work-groups
// per CU (at most 64, since a segment merges every earlier segment's pairs),
// and at least sqrt(pages) / 2 groups (a walk step costs a few merges, so
// steps and merges balance there: at 32 heads of 4K tokens one-group segments
// took 145 us and three-group ones 98),
// no more tokens than prefill_top_kernel holds (8K), and page slots enough for the
// segment's pairs (12 P bytes). One segment when the heads alone fill the GPU.
int prefill_segment(const Arena& a, int max_pages, int cus) {
  if (max_pages <= 1 || a.P == 0) return max(max_pages, 1);
  const size_t f = (size_t(a.page_bytes) - 8 * size_t(a.G)) & ~size_t(7);
  const int smin = int((12 * size_t(a.P) + f - 1) / f);
  const int smax = kTopPerThread * kTopThreads / a.G;
  if (smin > smax) return max_pages;
  const int64_t heads = int64_t(a.B) * a.Hkv;
  const int64_t want = std::min<int64_t>(64, std::max<int64_t>(1, 4 * int64_t(cus) / heads));
  if (want == 1) return max_pages;
  const int balance = int(std::ceil(std::sqrt(double(max_pages)) / 2));
  const int seg = std::max(int((max_pages + want - 1) / want), balance);
  return std::min(std::max(seg, smin), smax);
}

hipError_t launch_prefill(const Arena& a, const void* k, const void* v, int64_t max_len,
                          const PrefillLens& lens, int max_pages, hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const size_t lds_sel = prefill_select_lds_bytes(a.G, a.P);
  if (lds_sel > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_select_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(lds_sel));
    if (e != hipSuccess) return e;
  }
  const size_t lds_pack = pack_lds_bytes();
  const int slices = a.G > 128 ? a.G / 128 : 1;
  const __half* kh = static_cast<const __half*>(k);
  const __half* vh = static_cast<const __half*>(v);
  if (max_pages > 0) {
    hipLaunchKernelGGL(prefill_norms_kernel, dim3(max_pages, a.Hkv, a.B), dim3(a.G),
                       size_t(a.G) * 9 * sizeof(uint4), s, a, kh, max_len, lens);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int seg = prefill_segment(a, max_pages, cus);
  const int nseg = max_pages > 0 ? (max_pages + seg - 1) / seg : 1;
  if (nseg > 1) {
    hipLaunchKernelGGL(prefill_top_kernel, dim3(nseg - 1, a.Hkv, a.B), dim3(kTopThreads), 0, s,
                       a, lens, seg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prefill_select_kernel, dim3(nseg, a.Hkv, a.B), dim3(kWalkThreads), lds_sel,
                     s, a, kh, vh, max_len, lens, seg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_pages == 0) return e;
  if (slices == 2)
    hipLaunchKernelGGL(prefill_pack_kernel<2>, dim3(32 * ((max_pages + 7) / 8), a.Hkv, a.B),
                       dim3(kPackThreads), lds_pack, s, a, kh, vh, max_len, lens);
  else
    hipLaunchKernelGGL(prefill_pack_kernel<1>, dim3(2 * max_pages, a.Hkv, a.B),
                       dim3(kPackThreads), lds_pack, s, a, kh, vh, max_len, lens);
  return hipGetLastError();
}

hipError_t launch_quantize(const Arena& a, const QuantizeList& due, hipStream_t s) {
  dim3 grid(a.Hkv, due.n);
  // every candidate's rows resident in LDS when they fit the device's limit
  const size_t lds_res = resident_lds_bytes(a.G, a.P);
  const bool resident = a.lds_max > 0 && lds_res <= size_t(a.lds_max);
  const size_t lds = resident ? lds_res : quantize_lds_bytes(a.G, a.P);
  const void* fn = resident ? reinterpret_cast<const void*>(quantize_kernel<true>)
                            : reinterpret_cast<const void*>(quantize_kernel<false>);
  if (lds > 65536) {  // above the default dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  if (resident)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(kQuantThreads), lds, s, a, due);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(kQuantThreads), lds, s, a, due);
  return hipGetLastError();
}

}  // namespace ott
