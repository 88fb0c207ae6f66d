// Device-side arena addressing shared by the OTT kernels (gfx950).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ott_kernels.h"

namespace ott {
namespace dev {

constexpr int D = kHeadDim;
constexpr int kRingFlag = 0x40000000;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int32_t* counters(const Arena& a, int bh) {
  return reinterpret_cast<int32_t*>(a.base + a.off_counters) + size_t(bh) * 4;
}
// splits of the running decode done with head bh (0 between launches); taken
// and cleared with device-coherent atomics
__device__ __forceinline__ uint32_t* ticket(const Arena& a, int bh) {
  return reinterpret_cast<uint32_t*>(a.base + a.off_tickets) + bh;
}
__device__ __forceinline__ void reset_ticket(const Arena& a, int bh) {
  __hip_atomic_store(ticket(a, bh), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

}  // namespace dev
}  // namespace ott
