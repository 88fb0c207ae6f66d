// Internal interface between the host library (ott_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ott {

constexpr int kHeadDim = 128;
constexpr int kMaxBatch = 512;

// Device view of one handle's arena. Passed by value to every kernel.
struct Arena {
  uint8_t* base;
  int32_t B, Hq, Hkv, G, R, P, C;  // C = R + G (window ring capacity)
  int32_t nb_max;                  // pages per (sequence, KV head)
  int32_t max_splits;
  uint32_t page_bytes;
  uint64_t off_counters, off_pages, off_page_pos, off_page_nvalid;
  uint64_t off_pool_k, off_pool_v, off_pool_pos, off_pool_n2;
  uint64_t off_ring_k, off_ring_v, off_partials, off_tickets;
  float sm_scale;
  int32_t retention;  // pool rule: 0 smallest squared Key norm, 1 largest, 2 random per position
  int32_t lds_max;    // dynamic LDS bytes a work-group may use on this device (0: unknown)
};

// New-token counts of one ott_append call and the window slot of each
// sequence's first new token (known to the host, so the kernel's copies do
// not wait for a counter read); uint16 keeps the kernel argument at 2 KiB.
// init: the first launch on a handle whose counters no kernel has written yet
// (the arena's contents are unknown): every head's counters are set to
// {n, n, 0, 0} instead of being advanced.
struct AppendCounts {
  int32_t max_new;
  int32_t uniform;  // >= 0: every sequence appends this many; < 0: use n[]
  int32_t init;
  uint16_t n[kMaxBatch];
  uint16_t slot0[kMaxBatch];
};

// Which (sequence, KV head) work-group i of a one-split decode serves. The
// dispatcher places work-groups i, i + CUs, i + 2 CUs, ... on one CU, so the
// host orders heads by size to even out each CU's total (n = 0: identity).
constexpr int kMaxOrdered = 1024;
struct HeadOrder {
  int32_t n;
  uint16_t bh[kMaxOrdered];
};

hipError_t launch_append(const Arena& a, const void* k, const void* v, const AppendCounts& n,
                         hipStream_t s);
// The sequences whose window is full at an ott_quantize_group call.
// deferred = 0: the kernel checks the window is full and advances the counters.
// deferred = 1 (a fused step): the host has chosen the sequences; the kernel
// reads only the window head and page count, and the step's decode makes the
// new page visible (it applies the counter advance, see StepArgs).
struct QuantizeList {
  int32_t n;
  int32_t deferred;
  uint16_t b[kMaxBatch];
};
// The append half of a fused step (ott_step), carried by the decode launch:
// one new token per sequence, rows k/v [B][Hkv][D] (k == NULL: a plain decode).
// Sequences with their bit set in adv had a quantize step in this step: the
// decode first advances their counters (window head + G, window count - G,
// pages + 1). The new token is the last fp16 token the decode attends (read
// from k/v); the head's single writer (the one-split work-group, or the split
// merge) then stores it in window slot (head + r_cnt) % C and writes the counters.
struct StepArgs {
  const __half* k;
  const __half* v;
  uint32_t adv[kMaxBatch / 32];
};
hipError_t launch_quantize(const Arena& a, const QuantizeList& due, hipStream_t s);
// Prompt lengths of an ott_prefill call.
struct PrefillLens {
  int32_t len[kMaxBatch];
};
// k, v: fp16 [B][Hkv][max_len][D]; the cache must be empty; max_pages is the
// largest page count of any sequence (floor((L - R) / G) for L >= R + G).
hipError_t launch_prefill(const Arena& a, const void* k, const void* v, int64_t max_len,
                          const PrefillLens& lens, int max_pages, hipStream_t s);
hipError_t launch_decode(const Arena& a, const void* q, void* out, int num_splits,
                         const HeadOrder& order, const StepArgs& step, hipStream_t s);
// The decode kernel for a group of query heads per KV head (Hq > Hkv); it
// writes the output (one split) or the split partials like launch_decode.
hipError_t launch_decode_gqa(const Arena& a, const void* q, void* out, int num_splits,
                             const HeadOrder& order, const StepArgs& step, hipStream_t s);
// Work-groups of the decode kernel this arena's shape launches that fit on
// one CU at once (0 if the runtime cannot tell).
int decode_wgs_per_cu(const Arena& a);
int decode_gqa_wgs_per_cu(const Arena& a);

// The fp16 baseline decode: a plain fp16 KV cache [B][Hkv][max_len][D] and one
// query per (sequence, query head); part holds [B][Hq][S][2+D] split partials.
struct Fp16Cache {
  const __half* k;
  const __half* v;
  const __half* q;
  __half* out;
  float* part;
  int32_t B, Hq, Hkv, max_len;
  float sm_scale;
};
struct Fp16Lens {
  int32_t len[kMaxBatch];
};
// query heads of a KV head that share a loaded chunk (8, 4, 2 or 1)
int fp16_heads_per_pass(int nq);
// work-groups per CU of the fp16 kernel variant for hg heads per pass
int fp16_decode_wgs_per_cu(int hg);
hipError_t launch_fp16_decode(const Fp16Cache& c, const Fp16Lens& lens, int num_splits,
                              hipStream_t s);

// Dynamic LDS bytes the quantize kernel needs for (G, P).
size_t quantize_lds_bytes(int G, int P);

}  // namespace ott
