// Host side of the OTT C ABI: validation, arena map, host copies of the
// per-sequence counters, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/ott.h"
#include "ott_kernels.h"

struct ott_ctx {
  ott_config_t cfg;
  ott_layout_t lay;
  ott::Arena dev;
  std::vector<int32_t> L, rcnt, head, nb;  // identical for every KV head of a sequence
  int32_t forced_splits = 0;
  int64_t slots = 1024;  // decode work-groups the GPU holds at once
  int32_t cus = 256;     // compute units (work-group i and i + cus share a CU)
  ott::HeadOrder order{};  // rebuilt at every one-split decode
  ott::QuantizeList due{};  // rebuilt at every quantize call
  std::vector<int32_t> seq_by_size;
  std::vector<int32_t> ones;  // n_new of a step that falls back to the separate calls
  // pending[b]: ott_step already quantized sequence b's next group (page nb and
  // the other pool buffer are written, not yet visible); its due step's decode
  // makes them visible. Cleared by every call that changes state otherwise.
  std::vector<uint8_t> pending;
  bool counters_written = false;  // has a launch on this handle set every head's counters?
  bool poisoned = false;
};

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// the kernels move fp16 rows in 16-byte pieces
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

ott_status_t validate_config(const ott_config_t* c) {
  if (!c) return OTT_ERR_INVALID_ARG;
  if (c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1 || c->max_seq_len < 1 ||
      c->residual < 0 || c->pool_size < 0 || c->group_size < 1 || c->head_dim < 1)
    return OTT_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return OTT_ERR_INVALID_ARG;
  if (!(c->sm_scale == c->sm_scale)) return OTT_ERR_INVALID_ARG;  // NaN
  if (c->retention < OTT_RETAIN_SMALLEST_NORM || c->retention > OTT_RETAIN_RANDOM)
    return OTT_ERR_INVALID_ARG;
  if (c->batch > ott::kMaxBatch) return OTT_ERR_UNSUPPORTED;
  if (c->head_dim != ott::kHeadDim) return OTT_ERR_UNSUPPORTED;
  if (c->group_size != 64 && c->group_size != 128 && c->group_size != 256)
    return OTT_ERR_UNSUPPORTED;
  if (c->pool_size > 512 || c->residual > 4096) return OTT_ERR_UNSUPPORTED;
  const int nq = c->num_q_heads / c->num_kv_heads;
  if (nq > 64) return OTT_ERR_UNSUPPORTED;
  const int64_t heads = int64_t(c->batch) * c->num_kv_heads;
  if (heads > (1 << 20)) return OTT_ERR_UNSUPPORTED;
  if (c->num_kv_heads > 65535) return OTT_ERR_UNSUPPORTED;  // a grid dimension of the prefill
  return OTT_OK;
}

// Split-K capacity: enough partial slots for ~8K waves, 4..64 per head.
int max_splits_for(const ott_config_t* c) {
  const int64_t heads = int64_t(c->batch) * c->num_kv_heads;
  const int64_t s = (8192 + heads - 1) / heads;
  return int(std::max<int64_t>(4, std::min<int64_t>(64, s)));
}

void fill_layout(const ott_config_t* c, ott_layout_t* L) {
  const uint64_t B = c->batch, Hkv = c->num_kv_heads, Hq = c->num_q_heads, d = c->head_dim;
  const uint64_t G = c->group_size, P = c->pool_size, C = c->residual + c->group_size;
  const uint64_t BH = B * Hkv;
  const uint64_t NB = (uint64_t(c->max_seq_len) + G - 1) / G;
  *L = ott_layout_t{};
  L->page_bytes = G * d / 4 + d * G / 4 + 4 * d + 4 * G;
  L->pages_per_head = int32_t(NB);
  L->ring_capacity = int32_t(C);
  L->max_splits = max_splits_for(c);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L->off_counters = take(BH * 4 * sizeof(int32_t));
  L->off_pages = take(BH * NB * L->page_bytes);
  L->off_page_pos = take(BH * NB * G * sizeof(int32_t));
  L->off_page_nvalid = take(BH * NB * sizeof(int32_t));
  L->off_pool_k = take(2 * BH * P * d * 2);
  L->off_pool_v = take(2 * BH * P * d * 2);
  L->off_pool_pos = take(2 * BH * P * sizeof(int32_t));
  L->off_pool_n2 = take(2 * BH * P * sizeof(double));
  L->off_ring_k = take(BH * C * d * 2);
  L->off_ring_v = take(BH * C * d * 2);
  L->off_partials = take(B * Hq * uint64_t(L->max_splits) * (2 + d) * sizeof(float));
  L->off_tickets = take(BH * sizeof(uint32_t));
  L->arena_bytes = off;
}

ott_status_t check_handle(ott_handle_t h) {
  if (!h) return OTT_ERR_INVALID_ARG;
  if (h->poisoned) return OTT_ERR_HIP;
  return OTT_OK;
}

ott_status_t after_launch(ott_handle_t h, hipError_t e) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    h->poisoned = true;
    return OTT_ERR_HIP;
  }
  return OTT_OK;
}

// Split count and head order of a decode over the host copy of the counters
// (plus the step's new token when step.k is set), then the launch.
ott_status_t launch_decode_planned(ott_handle_t h, const void* d_q, void* d_out,
                                   const ott::StepArgs& step, void* stream) {
  const int B = h->cfg.batch;
  const int64_t extra = step.k ? 1 : 0;
  auto bytes = [&](int b) {
    const int64_t pc = std::min<int64_t>(h->cfg.pool_size, int64_t(h->cfg.group_size) * h->nb[b]);
    return int64_t(h->nb[b]) * int64_t(h->lay.page_bytes) +
           (pc + h->rcnt[b] + extra) * 4 * h->cfg.head_dim;
  };
  // bytes of the largest head (pages + fp16 tokens) bound the useful split count
  int64_t bytes_max = 0;
  for (int b = 0; b < B; ++b) bytes_max = std::max<int64_t>(bytes_max, bytes(b));
  int S = h->forced_splits;
  if (S <= 0) {
    // as many work-groups as the GPU holds at once, each with at least ~3
    // pages of work
    const int64_t heads = int64_t(B) * h->cfg.num_kv_heads;
    S = int(std::max<int64_t>(1, h->slots / heads));
    S = int(std::min<int64_t>(S, std::max<int64_t>(1, bytes_max / (3 * int64_t(h->lay.page_bytes)))));
  }
  S = std::max(1, std::min(S, h->dev.max_splits));
  // One split per head and heads of unequal size: deal the heads to CUs
  // largest first, in snake order over the rounds of `cus` work-groups, so
  // that each CU's total is about the same.
  ott::HeadOrder& ord = h->order;
  ord.n = 0;
  const int Hkv = h->cfg.num_kv_heads;
  const int64_t heads = int64_t(B) * Hkv;
  // (only whole rounds: a partial last round would leave holes in the order)
  if (S == 1 && heads <= ott::kMaxOrdered && heads > h->cus && heads % h->cus == 0) {
    std::vector<int32_t>& seq = h->seq_by_size;
    seq.resize(B);
    for (int b = 0; b < B; ++b) seq[b] = b;
    std::stable_sort(seq.begin(), seq.end(), [&](int x, int y) { return bytes(x) > bytes(y); });
    const int64_t C = h->cus;
    int64_t p = 0;
    for (int b : seq) {
      for (int hh = 0; hh < Hkv; ++hh, ++p) {
        const int64_t r = p / C, i = p % C;
        const int64_t slot = r * C + ((r & 1) ? C - 1 - i : i);
        ord.bh[slot] = uint16_t(b * Hkv + hh);
      }
    }
    ord.n = int32_t(heads);
  }
  return after_launch(h, ott::launch_decode(h->dev, d_q, d_out, S, ord, step,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ott_status_t ott_init(const ott_config_t* cfg, void* d_arena, size_t arena_bytes,
                      size_t* required_bytes, ott_handle_t* out) {
  ott_status_t st = validate_config(cfg);
  if (st != OTT_OK) return st;
  ott_layout_t lay;
  fill_layout(cfg, &lay);
  if (required_bytes) *required_bytes = size_t(lay.arena_bytes);
  if (!d_arena) {
    if (out) return OTT_ERR_INVALID_ARG;  // creating a handle needs an arena
    if (!required_bytes) return OTT_ERR_INVALID_ARG;
    return OTT_OK;
  }
  if (!out) return OTT_ERR_INVALID_ARG;
  if (arena_bytes < lay.arena_bytes || (reinterpret_cast<uintptr_t>(d_arena) % kAlign) != 0)
    return OTT_ERR_ARENA_TOO_SMALL;

  ott_ctx* h = new (std::nothrow) ott_ctx();
  if (!h) return OTT_ERR_INVALID_ARG;
  h->cfg = *cfg;
  if (h->cfg.sm_scale <= 0.f) h->cfg.sm_scale = 1.0f / std::sqrt(float(cfg->head_dim));
  h->lay = lay;
  ott::Arena& a = h->dev;
  a.base = static_cast<uint8_t*>(d_arena);
  a.B = cfg->batch;
  a.Hq = cfg->num_q_heads;
  a.Hkv = cfg->num_kv_heads;
  a.G = cfg->group_size;
  a.R = cfg->residual;
  a.P = cfg->pool_size;
  a.C = cfg->residual + cfg->group_size;
  a.nb_max = lay.pages_per_head;
  a.max_splits = lay.max_splits;
  a.page_bytes = uint32_t(lay.page_bytes);
  a.off_counters = lay.off_counters;
  a.off_pages = lay.off_pages;
  a.off_page_pos = lay.off_page_pos;
  a.off_page_nvalid = lay.off_page_nvalid;
  a.off_pool_k = lay.off_pool_k;
  a.off_pool_v = lay.off_pool_v;
  a.off_pool_pos = lay.off_pool_pos;
  a.off_pool_n2 = lay.off_pool_n2;
  a.off_ring_k = lay.off_ring_k;
  a.off_ring_v = lay.off_ring_v;
  a.off_partials = lay.off_partials;
  a.off_tickets = lay.off_tickets;
  a.sm_scale = h->cfg.sm_scale;
  a.retention = h->cfg.retention;
  const size_t nb = size_t(cfg->batch);
  h->L.assign(nb, 0);
  h->rcnt.assign(nb, 0);
  h->head.assign(nb, 0);
  h->nb.assign(nb, 0);
  h->pending.assign(nb, 0);
  {
    // one round of decode work-groups fills the GPU: CUs x work-groups per CU
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    int wpc = ott::decode_wgs_per_cu(a);
    if (wpc <= 0) wpc = 4;
    h->slots = int64_t(cus) * wpc;
    h->cus = cus;
    // the LDS a quantize work-group may opt into (0 if the runtime cannot tell)
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess)
      lds = 0;
    a.lds_max = lds;
  }
  // Nothing is written to the arena here: the first ott_append or ott_prefill
  // launch sets every head's counters on the caller's stream.
  *out = h;
  return OTT_OK;
}

ott_status_t ott_append(ott_handle_t h, const void* d_k, const void* d_v, const int32_t* h_n_new,
                        int32_t max_new, void* stream) {
  ott_status_t st = check_handle(h);
  if (st != OTT_OK) return st;
  if (!h_n_new || max_new < 0) return OTT_ERR_INVALID_ARG;
  const int B = h->cfg.batch;
  const int C = h->dev.C;
  bool any = false, uniform = true;
  for (int b = 0; b < B; ++b) {
    const int n = h_n_new[b];
    if (n < 0 || n > max_new) return OTT_ERR_INVALID_ARG;
    if (n != h_n_new[0]) uniform = false;
    if (n > 0) any = true;
  }
  if (!any) return OTT_OK;
  if (!d_k || !d_v || misaligned16(d_k) || misaligned16(d_v)) return OTT_ERR_INVALID_ARG;
  for (int b = 0; b < B; ++b) {
    const int n = h_n_new[b];
    if (h->rcnt[b] + n > C) return OTT_ERR_CAPACITY;
    if (int64_t(h->L[b]) + n > h->cfg.max_seq_len) return OTT_ERR_CAPACITY;
  }
  std::fill(h->pending.begin(), h->pending.end(), 0);
  ott::AppendCounts cnt{};
  cnt.max_new = max_new;
  cnt.uniform = uniform ? h_n_new[0] : -1;
  cnt.init = h->counters_written ? 0 : 1;
  for (int b = 0; b < B; ++b) {
    cnt.n[b] = uint16_t(h_n_new[b]);
    cnt.slot0[b] = uint16_t((h->head[b] + h->rcnt[b]) % C);
  }
  st = after_launch(h, ott::launch_append(h->dev, d_k, d_v, cnt, static_cast<hipStream_t>(stream)));
  if (st != OTT_OK) return st;
  h->counters_written = true;
  for (int b = 0; b < B; ++b) {
    h->L[b] += h_n_new[b];
    h->rcnt[b] += h_n_new[b];
  }
  return OTT_OK;
}

ott_status_t ott_quantize_group(ott_handle_t h, void* stream, int32_t* n_seq_quantized) {
  ott_status_t st = check_handle(h);
  if (st != OTT_OK) return st;
  const int B = h->cfg.batch, C = h->dev.C, G = h->dev.G;
  ott::QuantizeList& due = h->due;
  due.n = 0;
  due.deferred = 0;
  for (int b = 0; b < B; ++b)
    if (h->rcnt[b] >= C) due.b[due.n++] = uint16_t(b);
  const int ready = due.n;
  if (n_seq_quantized) *n_seq_quantized = 0;
  if (ready == 0) return OTT_OK;
  std::fill(h->pending.begin(), h->pending.end(), 0);
  st = after_launch(h, ott::launch_quantize(h->dev, due, static_cast<hipStream_t>(stream)));
  if (st != OTT_OK) return st;
  for (int b = 0; b < B; ++b) {
    if (h->rcnt[b] >= C) {
      h->head[b] = (h->head[b] + G) % C;
      h->rcnt[b] -= G;
      h->nb[b] += 1;
    }
  }
  if (n_seq_quantized) *n_seq_quantized = ready;
  return OTT_OK;
}

ott_status_t ott_prefill(ott_handle_t h, const void* d_k, const void* d_v, const int32_t* h_len,
                         int32_t max_len, void* stream) {
  ott_status_t st = check_handle(h);
  if (st != OTT_OK) return st;
  if (!h_len || max_len < 0) return OTT_ERR_INVALID_ARG;
  const int B = h->cfg.batch, G = h->cfg.group_size, R = h->cfg.residual, C = h->dev.C;
  ott::PrefillLens lens;
  bool any = false;
  for (int b = 0; b < B; ++b) {
    if (h->L[b] != 0) return OTT_ERR_STATE;  // prefill starts from an empty cache
    if (h_len[b] < 0 || h_len[b] > max_len) return OTT_ERR_INVALID_ARG;
    if (h_len[b] > h->cfg.max_seq_len) return OTT_ERR_CAPACITY;
    lens.len[b] = h_len[b];
    any |= h_len[b] > 0;
  }
  if (!any) return OTT_OK;
  if (!d_k || !d_v || misaligned16(d_k) || misaligned16(d_v)) return OTT_ERR_INVALID_ARG;
  std::fill(h->pending.begin(), h->pending.end(), 0);
  int max_pages = 0;
  for (int b = 0; b < B; ++b)
    if (h_len[b] >= R + G) max_pages = std::max(max_pages, (h_len[b] - R) / G);
  st = after_launch(h, ott::launch_prefill(h->dev, d_k, d_v, max_len, lens, max_pages,
                                           static_cast<hipStream_t>(stream)));
  if (st != OTT_OK) return st;
  h->counters_written = true;  // the pool walk sets every head's counters, empty ones included
  for (int b = 0; b < B; ++b) {
    const int L = h_len[b];
    const int nq = L >= R + G ? (L - R) / G : 0;
    h->L[b] = L;
    h->rcnt[b] = L - G * nq;
    h->head[b] = (G * nq) % C;
    h->nb[b] = nq;
  }
  return OTT_OK;
}

ott_status_t ott_decode(ott_handle_t h, const void* d_q, void* d_out, void* stream) {
  ott_status_t st = check_handle(h);
  if (st != OTT_OK) return st;
  if (!d_q || !d_out || misaligned16(d_q) || misaligned16(d_out)) return OTT_ERR_INVALID_ARG;
  for (int b = 0; b < h->cfg.batch; ++b)
    if (h->L[b] == 0) return OTT_ERR_STATE;
  ott::StepArgs step{};
  return launch_decode_planned(h, d_q, d_out, step, stream);
}

ott_status_t ott_step(ott_handle_t h, const void* d_k, const void* d_v, const void* d_q,
                      void* d_out, void* stream, int32_t* n_seq_quantized) {
  ott_status_t st = check_handle(h);
  if (st != OTT_OK) return st;
  if (!d_k || !d_v || !d_q || !d_out || misaligned16(d_k) || misaligned16(d_v) ||
      misaligned16(d_q) || misaligned16(d_out))
    return OTT_ERR_INVALID_ARG;
  const int B = h->cfg.batch, C = h->dev.C, G = h->dev.G, R = h->dev.R;
  for (int b = 0; b < B; ++b) {
    if (h->rcnt[b] >= C) return OTT_ERR_STATE;  // a full window: ott_quantize_group first
    if (int64_t(h->L[b]) + 1 > h->cfg.max_seq_len) return OTT_ERR_CAPACITY;
  }
  if (n_seq_quantized) *n_seq_quantized = 0;
  if (R == 0 || !h->counters_written) {
    // With R = 0 the new token belongs to the group a full window quantizes;
    // before any launch the counters are not set yet: the separate calls.
    h->ones.assign(size_t(B), 1);
    st = ott_append(h, d_k, d_v, h->ones.data(), 1, stream);
    if (st != OTT_OK) return st;
    st = ott_quantize_group(h, stream, n_seq_quantized);
    if (st != OTT_OK) return st;
    return ott_decode(h, d_q, d_out, stream);
  }
  // A window holding C - 1 tokens is full after this step's append: its group
  // (the G oldest tokens) is quantized and this step's decode makes the page
  // visible. With R >= 1 the group never includes the new token, and it is
  // complete as soon as the window holds G tokens, R - 1 steps or more before
  // it is due: the quantize step may run any time in between, writing only
  // what no decode reads yet (page nb, the other pool buffer) and reading what
  // no append writes (the group's window slots, the live pool). So when some
  // window is due and not quantized yet, one launch quantizes every window
  // whose group is complete; the others' pages wait for their due steps.
  ott::StepArgs step{};
  step.k = static_cast<const __half*>(d_k);
  step.v = static_cast<const __half*>(d_v);
  bool launch = false;
  int n_due = 0;
  for (int b = 0; b < B; ++b) {
    if (h->rcnt[b] + 1 >= C) {
      ++n_due;
      step.adv[b >> 5] |= 1u << (b & 31);
      launch |= !h->pending[b];
    }
  }
  if (launch) {
    ott::QuantizeList& batch = h->due;
    batch.n = 0;
    batch.deferred = 1;
    for (int b = 0; b < B; ++b)
      if (h->rcnt[b] >= G && !h->pending[b]) batch.b[batch.n++] = uint16_t(b);
    st = after_launch(h, ott::launch_quantize(h->dev, batch, static_cast<hipStream_t>(stream)));
    if (st != OTT_OK) return st;
    for (int i = 0; i < batch.n; ++i) h->pending[batch.b[i]] = 1;
  }
  // the host copy of the counters as the decode sees them (the due pages
  // visible, before the append), then after the append
  for (int b = 0; b < B; ++b) {
    if (h->rcnt[b] + 1 >= C) {
      h->head[b] = (h->head[b] + G) % C;
      h->rcnt[b] -= G;
      h->nb[b] += 1;
      h->pending[b] = 0;
    }
  }
  st = launch_decode_planned(h, d_q, d_out, step, stream);
  for (int b = 0; b < B; ++b) {
    h->L[b] += 1;
    h->rcnt[b] += 1;
  }
  if (st == OTT_OK && n_seq_quantized) *n_seq_quantized = n_due;
  return st;
}

void ott_destroy(ott_handle_t h) { delete h; }

ott_status_t ott_get_layout(ott_handle_t h, ott_layout_t* out) {
  if (!h || !out) return OTT_ERR_INVALID_ARG;
  *out = h->lay;
  return OTT_OK;
}

ott_status_t ott_get_seq_state(ott_handle_t h, int32_t b, int32_t out[4]) {
  if (!h || !out || b < 0 || b >= h->cfg.batch) return OTT_ERR_INVALID_ARG;
  out[0] = h->L[b];
  out[1] = h->rcnt[b];
  out[2] = h->head[b];
  out[3] = h->nb[b];
  return OTT_OK;
}

ott_status_t ott_set_num_splits(ott_handle_t h, int32_t num_splits) {
  if (!h || num_splits < 0 || num_splits > h->lay.max_splits) return OTT_ERR_INVALID_ARG;
  h->forced_splits = num_splits;
  return OTT_OK;
}

}  // extern "C"

namespace {

// Work-groups of the fp16 baseline kernel the current device holds at once
// (CUs x work-groups per CU), per device and heads-per-pass variant, asked of
// the runtime once: the answer does not change while the process runs.
int64_t fp16_decode_slots(int hg) {
  constexpr int kDevices = 64;
  static std::atomic<int64_t> cache[kDevices][9];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) dev = -1;
  if (dev >= 0) {
    const int64_t c = cache[dev][hg].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int wpc = ott::fp16_decode_wgs_per_cu(hg);
  if (wpc <= 0) wpc = 2;
  const int64_t slots = int64_t(cus) * wpc;
  if (dev >= 0) cache[dev][hg].store(slots, std::memory_order_relaxed);
  return slots;
}

}  // namespace

namespace {

// Split workspace of ott_fp16_decode_noalloc, owned by the library: each GPU
// the library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[OTT_FP16_DECODE_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchDevices];  // per device; looked up once, with that device current

// Device address of the current device's copy of `scratch` (NULL if the
// runtime cannot tell).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

// ott_fp16_decode with its split partials in d_work (work_bytes of it), or,
// when scratch_addr is given, in the library's scratch (work_bytes = its size;
// too many splits is OTT_ERR_SCRATCH_TOO_SMALL instead of
// OTT_ERR_ARENA_TOO_SMALL). Arguments are validated before any HIP call.
ott_status_t fp16_decode_on(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, const void* d_k, const void* d_v, int32_t max_len,
                            const int32_t* h_len, const void* d_q, void* d_out, float sm_scale,
                            void* d_work, size_t work_bytes, int32_t num_splits, void* stream,
                            void* (*scratch_addr)()) {
  if (batch < 1 || batch > ott::kMaxBatch || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
      num_q_heads % num_kv_heads != 0 || max_len < 1 || num_splits < 0 || !h_len)
    return OTT_ERR_INVALID_ARG;
  if (head_dim != ott::kHeadDim) return OTT_ERR_UNSUPPORTED;
  if (!d_k || !d_v || !d_q || !d_out) return OTT_ERR_INVALID_ARG;
  if (misaligned16(d_k) || misaligned16(d_v) || misaligned16(d_q) || misaligned16(d_out))
    return OTT_ERR_INVALID_ARG;
  ott::Fp16Lens lens;
  int32_t lmax = 0;
  for (int b = 0; b < batch; ++b) {
    if (h_len[b] < 1 || h_len[b] > max_len) return OTT_ERR_STATE;
    lens.len[b] = h_len[b];
    lmax = std::max(lmax, h_len[b]);
  }
  // splits: as given, or enough work-groups for one round of the GPU with at
  // least 256 tokens each; never more than the workspace holds
  const bool library_scratch = scratch_addr != nullptr;
  const size_t per_split = size_t(batch) * num_q_heads * (2 + ott::kHeadDim) * sizeof(float);
  const int64_t fit = (d_work == nullptr && !library_scratch) ? 1 : int64_t(work_bytes / per_split);
  int S = num_splits;
  if (S == 0) {
    const int64_t slots = fp16_decode_slots(ott::fp16_heads_per_pass(num_q_heads / num_kv_heads));
    S = int(std::max<int64_t>(1, slots / (int64_t(batch) * num_kv_heads)));
    S = int(std::min<int64_t>(S, std::max<int64_t>(1, (lmax + 255) / 256)));
    S = int(std::min<int64_t>(S, std::max<int64_t>(1, fit)));
  } else if (S > 1 && S > fit) {
    return library_scratch ? OTT_ERR_SCRATCH_TOO_SMALL : OTT_ERR_ARENA_TOO_SMALL;
  }
  void* part = d_work;
  if (library_scratch && S > 1) {
    part = scratch_addr();
    if (part == nullptr) return OTT_ERR_HIP;
  }
  ott::Fp16Cache c;
  c.k = static_cast<const __half*>(d_k);
  c.v = static_cast<const __half*>(d_v);
  c.q = static_cast<const __half*>(d_q);
  c.out = static_cast<__half*>(d_out);
  c.part = static_cast<float*>(part);
  c.B = batch;
  c.Hq = num_q_heads;
  c.Hkv = num_kv_heads;
  c.max_len = max_len;
  c.sm_scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(float(head_dim));
  return ott::launch_fp16_decode(c, lens, S, static_cast<hipStream_t>(stream)) == hipSuccess
             ? OTT_OK
             : OTT_ERR_HIP;
}

}  // namespace

extern "C" {

size_t ott_fp16_decode_workspace(int32_t batch, int32_t num_q_heads, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || num_splits <= 1) return 0;
  return size_t(batch) * num_q_heads * num_splits * (2 + ott::kHeadDim) * sizeof(float);
}

ott_status_t ott_fp16_decode(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, const void* d_k, const void* d_v, int32_t max_len,
                             const int32_t* h_len, const void* d_q, void* d_out, float sm_scale,
                             void* d_work, size_t work_bytes, int32_t num_splits, void* stream) {
  return fp16_decode_on(batch, num_q_heads, num_kv_heads, head_dim, d_k, d_v, max_len, h_len, d_q,
                        d_out, sm_scale, d_work, work_bytes, num_splits, stream, nullptr);
}

ott_status_t ott_fp16_decode_noalloc(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, const void* d_k, const void* d_v,
                                     int32_t max_len, const int32_t* h_len, const void* d_q,
                                     void* d_out, float sm_scale, int32_t num_splits,
                                     void* stream) {
  return fp16_decode_on(batch, num_q_heads, num_kv_heads, head_dim, d_k, d_v, max_len, h_len, d_q,
                        d_out, sm_scale, nullptr, OTT_FP16_DECODE_SCRATCH_BYTES, num_splits,
                        stream, scratch_on_current_device);
}

const char* ott_status_string(ott_status_t s) {
  switch (s) {
    case OTT_OK: return "ok";
    case OTT_ERR_INVALID_ARG: return "invalid argument";
    case OTT_ERR_UNSUPPORTED: return "unsupported configuration";
    case OTT_ERR_ARENA_TOO_SMALL: return "arena too small or misaligned";
    case OTT_ERR_CAPACITY: return "window or sequence capacity exceeded";
    case OTT_ERR_STATE: return "invalid state for this call";
    case OTT_ERR_HIP: return "HIP error (handle poisoned)";
    case OTT_ERR_SCRATCH_TOO_SMALL:
      return "request exceeds the library's fixed scratch (OTT_FP16_DECODE_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
