// Baseline decode over an uncompressed fp16 KV cache (gfx950, wave64).
//
// The pages measure OTT's decode throughput against the model running on its
// ordinary FP16 KV cache ([Abs] sciencestack.ai, Figure 3(a); [Blog]
// zijie-tian.site summary, section 4: 2.3x at batch 32). This kernel is that
// comparison point on the same shapes: out = softmax(sm_scale q K^T) V for one
// query per (sequence, query head) over the sequence's len fp16 rows of K and V.
//
// Work-group = 4 waves on one (sequence, KV head, split); a split is a range of
// 16-token chunks. The waves take chunks round-robin with the next chunk's
// rows in flight while the current one is attended; HG query heads of the KV
// head share every loaded chunk. The four wave states merge in LDS; with more
// than one split the partial states go to the caller's workspace and a second
// kernel merges them.
#include "ott_decode_common.h"

namespace ott {
namespace {
using namespace dev;
using namespace dec;

__device__ __forceinline__ void load_chunk(const __half* __restrict__ kb,
                                           const __half* __restrict__ vb, int base, int cnt,
                                           Fp16Rows& r, int lane) {
  const int rw = lane >> 4, c8 = lane & 15;
  // rows past the sequence read its last row (in bounds); fp16_attend gives
  // them weight zero
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p)
    r.k[p] = ld_nt4(kb + size_t(base + min(4 * p + rw, cnt - 1)) * D + 8 * c8);
#pragma unroll
  for (int p = 0; p < kF16Pass; ++p)
    r.v[p] = ld_nt4(vb + size_t(base + min(4 * p + rw, cnt - 1)) * D + 8 * c8);
}

template <int HG>
__global__ __launch_bounds__(256) void fp16_decode_kernel(Fp16Cache c, Fp16Lens lens, int S) {
  __shared__ float fin[kWaves][HG][D];
  __shared__ float mg_m[kWaves][HG], mg_l[kWaves][HG];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x % S, bh = blockIdx.x / S;
  const int b = bh / c.Hkv, hk = bh % c.Hkv;
  const int len = lens.len[b];
  const int nch = (len + kF16Chunk - 1) / kF16Chunk;
  const int ch0 = int(int64_t(s) * nch / S), ch1 = int(int64_t(s + 1) * nch / S);
  const int NQ = c.Hq / c.Hkv;
  const __half* kb = c.k + size_t(bh) * c.max_len * D;
  const __half* vb = c.v + size_t(bh) * c.max_len * D;
  const float qscale = c.sm_scale * kLog2e;

  for (int q0 = 0; q0 < NQ; q0 += HG) {
    const int qh0 = hk * NQ + q0;
    uint4 q8[HG];
    Fp16State st[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      q8[h] = reinterpret_cast<const uint4*>(c.q + (size_t(b) * c.Hq + qh0 + h) * D)[lane & 15];
      st[h].m = -INFINITY;
      st[h].l = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) st[h].acc[e] = 0.f;
    }
    int ch = ch0 + wave;
    Fp16Rows cur, nxt;
    if (ch < ch1) load_chunk(kb, vb, ch * kF16Chunk, min(kF16Chunk, len - ch * kF16Chunk), cur, lane);
    for (; ch < ch1; ch += kWaves) {
      const int cn = ch + kWaves;
      if (cn < ch1) load_chunk(kb, vb, cn * kF16Chunk, min(kF16Chunk, len - cn * kF16Chunk), nxt, lane);
      const int cnt = min(kF16Chunk, len - ch * kF16Chunk);
#pragma unroll
      for (int h = 0; h < HG; ++h) fp16_attend(cur, cnt, q8[h], qscale, st[h], lane);
      cur = nxt;
    }
    // wave state -> LDS: the four token rows (lane >> 4) of every channel add up
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float lt = wave_sum(st[h].l);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f32x2 p = swap16(st[h].acc[e]);
        const float x = p.x + p.y;
        p = swap32(x);
        v[e] = p.x + p.y;
      }
      if (lane < 16) {
        float4* f = reinterpret_cast<float4*>(&fin[wave][h][8 * lane]);
        f[0] = make_float4(v[0], v[1], v[2], v[3]);
        f[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
      if (lane == 0) {
        mg_m[wave][h] = st[h].m;
        mg_l[wave][h] = lt;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < HG * D; x += blockDim.x) {
      const int h = x / D, cc = x % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mg_m[w][h]);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = (mg_m[w][h] == -INFINITY) ? 0.f : exp2f(mg_m[w][h] - M);
        Ls = fmaf(mg_l[w][h], f, Ls);
        A = fmaf(fin[w][h][cc], f, A);
      }
      const size_t bq = size_t(b) * c.Hq + qh0 + h;
      if (S == 1) {
        c.out[bq * D + cc] = __float2half_rn(A / Ls);
      } else {
        float* part = c.part + (bq * S + s) * (2 + D);
        part[2 + cc] = A;
        if (cc == 0) {
          part[0] = M;
          part[1] = Ls;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(D) void fp16_combine_kernel(Fp16Cache c, int S) {
  const size_t bq = blockIdx.x;
  c.out[bq * D + threadIdx.x] =
      __float2half_rn(merge_partials(c.part + bq * S * (2 + D), S, threadIdx.x));
}

template <int HG>
hipError_t launch_hg(const Fp16Cache& c, const Fp16Lens& lens, int S, hipStream_t st) {
  hipLaunchKernelGGL(fp16_decode_kernel<HG>, dim3(unsigned(c.B) * c.Hkv * S), dim3(64 * kWaves), 0,
                     st, c, lens, S);
  return hipGetLastError();
}

template <int HG>
int wgs_hg() {
  int n = 0;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fp16_decode_kernel<HG>, 64 * kWaves, 0) ==
                 hipSuccess
             ? n
             : 0;
}

}  // namespace

int fp16_heads_per_pass(int nq) { return nq % 8 == 0 ? 8 : nq % 4 == 0 ? 4 : nq % 2 == 0 ? 2 : 1; }

int fp16_decode_wgs_per_cu(int hg) {
  switch (hg) {
    case 8: return wgs_hg<8>();
    case 4: return wgs_hg<4>();
    case 2: return wgs_hg<2>();
    default: return wgs_hg<1>();
  }
}

hipError_t launch_fp16_decode(const Fp16Cache& c, const Fp16Lens& lens, int S, hipStream_t st) {
  hipError_t e;
  switch (fp16_heads_per_pass(c.Hq / c.Hkv)) {
    case 8: e = launch_hg<8>(c, lens, S, st); break;
    case 4: e = launch_hg<4>(c, lens, S, st); break;
    case 2: e = launch_hg<2>(c, lens, S, st); break;
    default: e = launch_hg<1>(c, lens, S, st); break;
  }
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(fp16_combine_kernel, dim3(unsigned(c.B) * c.Hq), dim3(D), 0, st, c, S);
  return hipGetLastError();
}

}  // namespace ott
