/*
 * ott.h - C ABI of the MI355X (gfx950) Outlier Tokens Tracing decode-attention library.
 *
 * The method: "Accurate KV Cache Quantization with Outlier Tokens Tracing"
 * (arXiv 2505.10938). Passages are cited by page and section:
 *   [Blog] zijie-tian.site summary page: section 3.1 (group quantization every G
 *          tokens, Key-norm outlier rule), 3.2 (Outlier Pool), 3.3 (three caches,
 *          one fused decode) and its flowchart; section 4 (defaults G=128, R=32).
 *   [Abs]  sciencestack.ai page: TL;DR; Abstract (Keys per channel, Values per
 *          token); Figure 1(c) (smallest Key magnitude is the retention rule);
 *          Figure 2 (decoding stage on top, quantization stage below).
 *
 * One handle serves one attention layer: B sequences, Hkv KV heads, Hq query
 * heads (Hq a multiple of Hkv), head_dim 128. Each (sequence, KV head) owns
 *   - a 2-bit quantized cache of pages, one page per quantized group,
 *   - an outlier pool of up to P fp16 tokens (smallest squared Key L2 norm),
 *   - an fp16 residual window (a ring of R+G slots) of unquantized tokens.
 * A decode step is: ott_append (one token per sequence), ott_quantize_group
 * (a no-op unless some window is full), ott_decode.
 *
 * Ownership: the caller owns all device memory - the arena and every input and
 * output buffer. The library allocates no device memory and never synchronizes
 * a stream; it only enqueues kernels on the stream it is given. The host
 * handle is the library's; ott_destroy frees it.
 * Errors: every call returns a status and validates its arguments before it
 * enqueues anything, so a rejected call leaves the state unchanged. A failed
 * kernel launch poisons the handle: later calls return OTT_ERR_HIP.
 * Threading: a handle is not thread-safe; calls on one handle must be issued
 * in order, on one stream or with the caller ordering the streams.
 * Streams are passed as `void*` holding a hipStream_t (NULL = default stream).
 */
#ifndef OTT_H_
#define OTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ott_ctx* ott_handle_t;

typedef enum {
  OTT_OK = 0,
  OTT_ERR_INVALID_ARG = 1,     /* NULL pointer, out-of-range value */
  OTT_ERR_UNSUPPORTED = 2,     /* valid but not built: head_dim != 128, G not 64/128/256, ... */
  OTT_ERR_ARENA_TOO_SMALL = 3, /* arena_bytes below the required size, or misaligned arena */
  OTT_ERR_CAPACITY = 4,        /* append would overflow the window or max_seq_len */
  OTT_ERR_STATE = 5,           /* decode of a sequence that holds no token */
  OTT_ERR_HIP = 6,             /* a HIP launch failed; the handle is poisoned */
  OTT_ERR_SCRATCH_TOO_SMALL = 7 /* the request needs more than the library's fixed scratch */
} ott_status_t;

/* Layer shape and OTT hyper-parameters ([Blog] 3.1-3.3, section 4 and 6). */
typedef struct {
  int32_t batch;        /* B, 1..512 */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv with Hq/Hkv <= 64 */
  int32_t num_kv_heads; /* Hkv, 1..65535; B * Hkv <= 2^20 */
  int32_t head_dim;     /* d, must be 128 */
  int32_t group_size;   /* G: tokens per quantized group, 64, 128 or 256 */
  int32_t residual;     /* R >= 0: tokens always kept in the fp16 window */
  int32_t pool_size;    /* P, 0..512: outlier-pool capacity (0 = plain 2-bit cache) */
  int32_t max_seq_len;  /* tokens a sequence may reach, >= 1 */
  float sm_scale;       /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t retention;    /* which tokens the pool keeps: OTT_RETAIN_* (0 = the method's rule) */
} ott_config_t;

/*
 * Pool retention rules. The method keeps the P tokens with the smallest Key
 * magnitude ([Abs] TL;DR and Figure 1(c); [Blog] 3.1): squared L2 norm, fp64,
 * summed over channels 0..d-1. Figure 1(c) compares that choice with others; two
 * are built for that comparison. Each candidate gets a key and the pool keeps
 * the P smallest keys, ties to the lower position:
 *   OTT_RETAIN_SMALLEST_NORM  key = squared norm
 *   OTT_RETAIN_LARGEST_NORM   key = -squared norm
 *   OTT_RETAIN_RANDOM         key = (splitmix64(position) >> 11) * 2^-53, where
 *                             splitmix64(s) is the first output of a SplitMix64
 *                             generator with state s (Vigna's reference form)
 * pool_n2 holds the keys.
 */
enum { OTT_RETAIN_SMALLEST_NORM = 0, OTT_RETAIN_LARGEST_NORM = 1, OTT_RETAIN_RANDOM = 2 };

/*
 * Arena map (byte offsets from the arena base; every region is 256-byte aligned).
 * "bh" is b*Hkv + kvh. "NB" is pages_per_head = ceil(max_seq_len / G).
 *   counters   int32 [B*Hkv][4]: {L, r_cnt, ring_head, nb} of each (sequence, KV head)
 *   pages      [B*Hkv][NB][page_bytes], page n = the n-th quantized group, laid out as
 *                K codes  [G tokens][d/4 bytes], token-major: byte j of token t holds
 *                         channels 4j..4j+3, channel 4j+i in bits 2i..2i+1;
 *                V codes  [d channels][G/4 bytes], channel-major: byte j of channel c
 *                         holds slots 4j..4j+3, slot 4j+i in bits 2i..2i+1;
 *                K meta   [d] x {fp16 min, fp16 scale}   (per channel, [Abs] Abstract);
 *                V meta   [G] x {fp16 min, fp16 scale}   (per token,  [Abs] Abstract);
 *              members are in position order, slots >= n_valid are all-zero bytes.
 *              page_bytes = G*d/4 + d*G/4 + 4*d + 4*G (9216 at G=128, d=128).
 *   page_pos   int32 [B*Hkv][NB][G]: member positions (-1 past n_valid); tests only
 *   page_nvalid int32 [B*Hkv][NB]: members per page; tests only
 *   pool_k, pool_v   fp16  [2][B*Hkv][P][d]
 *   pool_pos         int32 [2][B*Hkv][P]
 *   pool_n2          fp64  [2][B*Hkv][P]   retention key of each pool token (its squared Key
 *                                          norm under the method's rule)
 *              two buffers: after nb quantize steps the live pool is buffer (nb & 1);
 *              its first min(P, G*nb) slots are used, ascending (key, position).
 *   ring_k, ring_v   fp16  [B*Hkv][R+G][d]: the window; its r_cnt tokens sit in slots
 *              (ring_head + i) % (R+G), i = 0..r_cnt-1, at positions G*nb + i.
 *   partials   fp32  [B][Hq][max_splits][2+d]: split-K partial softmax states {m, l, acc[d]}
 *              (written by the splits of a decode, read by the split that merges them).
 *   tickets    uint32 [B*Hkv]: splits of the running decode done with each (sequence, KV
 *              head); 0 between launches (the merging split resets it; the first append or
 *              prefill on the handle writes the 0).
 * No region needs to be cleared by the caller: every byte a kernel reads was
 * written earlier by one of this handle's kernels.
 */
typedef struct {
  uint64_t arena_bytes;
  uint64_t page_bytes;
  int32_t pages_per_head;
  int32_t ring_capacity;
  int32_t max_splits;
  int32_t reserved0;
  uint64_t off_counters;
  uint64_t off_pages;
  uint64_t off_page_pos;
  uint64_t off_page_nvalid;
  uint64_t off_pool_k;
  uint64_t off_pool_v;
  uint64_t off_pool_pos;
  uint64_t off_pool_n2;
  uint64_t off_ring_k;
  uint64_t off_ring_v;
  uint64_t off_partials;
  uint64_t off_tickets;
} ott_layout_t;

/*
 * ott_init - validate a config, size the arena, and create a handle.
 *   Sizing: pass d_arena = NULL and out = NULL; *required_bytes receives the size.
 *   Create: pass a device arena of >= required bytes (256-byte aligned); *out
 *   receives the handle. The arena may hold anything: ott_init neither reads
 *   nor writes it and enqueues no work. The first ott_append or ott_prefill
 *   that launches a kernel sets every (sequence, head) counter on its own
 *   stream, so the caller's stream order covers the arena from the start.
 *   required_bytes may be NULL when creating.
 */
ott_status_t ott_init(const ott_config_t* cfg, void* d_arena, size_t arena_bytes,
                      size_t* required_bytes, ott_handle_t* out);

/*
 * ott_append - add new tokens to each sequence's fp16 window ([Blog] 3.3: the
 * residual window keeps recent tokens in FP16).
 *   d_k, d_v : device fp16 [B][Hkv][max_new][d], 16-byte aligned; token i of
 *              sequence b is row i and takes position L_b + i. Copied; reusable once
 *              the stream has run. NULL or misaligned: OTT_ERR_INVALID_ARG.
 *   h_n_new  : host int32 [B], 0 <= n_new[b] <= max_new.
 *   Fails with OTT_ERR_CAPACITY (nothing enqueued) when some r_cnt_b + n_new[b]
 *   exceeds R+G (call ott_quantize_group first) or L_b + n_new[b] > max_seq_len.
 */
ott_status_t ott_append(ott_handle_t h, const void* d_k, const void* d_v, const int32_t* h_n_new,
                        int32_t max_new, void* stream);

/*
 * ott_quantize_group - the quantization stage ([Blog] 3.1-3.2 and flowchart;
 * [Abs] Figure 2 bottom). For every sequence whose window holds R+G tokens, and
 * for each of its KV heads, one group is processed:
 *   the G oldest window tokens and the pool compete; the P with the smallest
 *   squared Key norm (fp64, summed over channels 0..d-1; ties to the lower
 *   position) form the new pool; every other candidate, evicted pool tokens
 *   included, is quantized to 2 bits as one new page:
 *     scale = fp16_rne(fp32(max - min) / 3), min stored as fp16,
 *     code  = clamp(rint_half_even(fp32(x - min) / scale), 0, 3) (0 when scale is 0),
 *   per channel over the members for Keys, per member over its d channels for Values.
 *   *n_seq_quantized (may be NULL) receives the number of sequences processed.
 *   A no-op (nothing enqueued) when no window is full.
 */
ott_status_t ott_quantize_group(ott_handle_t h, void* stream, int32_t* n_seq_quantized);

/*
 * ott_prefill - a whole prompt into an empty cache in one call, with exactly the
 * state that appending it token by token and running every due quantize step in
 * order would leave ([Blog] 3.1: the quantization stage runs every G tokens; the
 * prompt is processed group by group in position order, each group competing with
 * the pool the previous groups left). Sequence b gets floor((len - R) / G) pages
 * (0 when len < R + G) and its last len - G*pages tokens in the window.
 *   d_k, d_v : device fp16 [B][Hkv][max_len][d], 16-byte aligned; token i of
 *              sequence b is row i (position i).
 *   h_len    : host int32 [B], 0 <= h_len[b] <= max_len (else OTT_ERR_INVALID_ARG),
 *              h_len[b] <= max_seq_len (else OTT_ERR_CAPACITY).
 *   Every sequence must be empty (else OTT_ERR_STATE, nothing enqueued). Up to
 *   four launches: every group token's squared Key norm at once; when the heads
 *   alone do not fill the GPU, each segment of groups' P smallest (key, position)
 *   pairs (the pool after a step holds the P smallest of all groups so far); the
 *   pool walk, one work-group per (segment, sequence, KV head), groups in position
 *   order from the merge of the earlier segments' pairs; then every page at once.
 *   A no-op when every length is 0.
 */
ott_status_t ott_prefill(ott_handle_t h, const void* d_k, const void* d_v, const int32_t* h_len,
                         int32_t max_len, void* stream);
/*
 * ott_decode - the decoding stage ([Blog] flowchart and 3.3; [Abs] Figure 2 top).
 * For each sequence b and query head qh (KV head qh / (Hq/Hkv)):
 *   out = sum_i softmax_i(sm_scale * q.k_i) v_i over every cached token of b:
 *   dequantized page tokens (k = min + scale*code), the fp16 pool and the fp16
 *   window, with one softmax over all of them.
 *   d_q   : device fp16 [B][Hq][d];  d_out : device fp16 [B][Hq][d]; both 16-byte
 *           aligned (else OTT_ERR_INVALID_ARG).
 *   The state is not modified; the call can be repeated. One launch: with
 *   split-K (ott_set_num_splits) the last split of each head to finish merges
 *   the partial states in split order, so results do not depend on timing.
 *   Two decodes of one handle must not overlap in time (they share the arena's
 *   partials and tickets): order their streams like any other calls.
 *   OTT_ERR_STATE if some sequence holds no token.
 */
ott_status_t ott_decode(ott_handle_t h, const void* d_q, void* d_out, void* stream);

/*
 * ott_step - one whole decode step in as few launches as possible: the same
 * state and output as ott_append (one token per sequence), ott_quantize_group,
 * ott_decode ([Blog] flowchart: a quantization stage every G tokens, a decoding
 * stage every token; [Abs] Figure 2).
 *   d_k, d_v : device fp16 [B][Hkv][d], the new token of every sequence (position
 *              L_b); d_q, d_out : device fp16 [B][Hq][d]. All 16-byte aligned, else
 *              OTT_ERR_INVALID_ARG. The k/v rows are copied into the window.
 *   *n_seq_quantized (may be NULL) receives the number of sequences whose group
 *   was quantized in this step.
 *   How: with R >= 1 the group a full window quantizes (its G oldest tokens)
 *   never includes the new token and is complete once the window holds G
 *   tokens, so its quantize step can run early: when a window is due and its
 *   group not yet quantized, one launch quantizes every window whose group is
 *   complete, writing only the next page and the other pool buffer, which no
 *   decode reads until that window's due step; the due step's decode then makes
 *   the page visible (the result is the same as quantizing at the due step).
 *   The decode attends the new token from d_k/d_v and the head's single writer
 *   (its only split, or its last split to finish) stores it in the window. One
 *   launch per step, one more on the steps that quantize. With R = 0 (the new token joins the group) or
 *   before any append/prefill, the three calls are made.
 *   OTT_ERR_STATE if some window already holds R+G tokens (call
 *   ott_quantize_group first); OTT_ERR_CAPACITY if some L_b + 1 > max_seq_len.
 *   Nothing is enqueued on error.
 */
ott_status_t ott_step(ott_handle_t h, const void* d_k, const void* d_v, const void* d_q,
                      void* d_out, void* stream, int32_t* n_seq_quantized);

/* ott_destroy - free the host handle (the arena stays the caller's). NULL is a no-op. */
void ott_destroy(ott_handle_t h);

/* ott_get_layout - the arena map of a handle. */
ott_status_t ott_get_layout(ott_handle_t h, ott_layout_t* out);

/*
 * ott_get_seq_state - host copy of sequence b's counters:
 * out[0] = L (tokens), out[1] = r_cnt (window tokens), out[2] = ring_head,
 * out[3] = nb (pages). Every KV head of a sequence holds the same values.
 */
ott_status_t ott_get_seq_state(ott_handle_t h, int32_t b, int32_t out[4]);

/*
 * ott_set_num_splits - split-K factor of ott_decode: 0 = automatic, otherwise
 * 1..max_splits work-groups per (sequence, KV head). Results agree to rounding.
 */
ott_status_t ott_set_num_splits(ott_handle_t h, int32_t num_splits);

/*
 * ott_fp16_decode - the comparison point of the pages' throughput figure
 * ([Abs] Figure 3(a); [Blog] section 4: OTT decodes 2.3x faster than the model
 * on its ordinary FP16 KV cache at batch 32): single-query decode attention over
 * an uncompressed fp16 KV cache, no quantization, no pool, no window.
 * For each sequence b and query head qh (KV head qh / (Hq/Hkv)):
 *   out[b][qh] = sum_t softmax_t(sm_scale * q[b][qh] . k[b][kvh][t]) v[b][kvh][t],
 *   t = 0..h_len[b]-1.
 *   d_k, d_v   : device fp16 [batch][num_kv_heads][max_len][head_dim], 16-byte aligned;
 *                rows at and past h_len[b] are not read.
 *   h_len      : host int32 [batch], 1 <= h_len[b] <= max_len (else OTT_ERR_STATE).
 *   d_q, d_out : device fp16 [batch][num_q_heads][head_dim], 16-byte aligned.
 *   sm_scale   : <= 0 selects 1/sqrt(head_dim). head_dim must be 128 (else OTT_ERR_UNSUPPORTED).
 *   d_work     : caller-owned device workspace for split partials (may be NULL, then one
 *                split); work_bytes its size. num_splits: 0 = automatic (fits the workspace),
 *                1 = no workspace used, n > 1 needs ott_fp16_decode_workspace(batch, Hq, n)
 *                bytes (else OTT_ERR_ARENA_TOO_SMALL, nothing enqueued).
 * Stateless: no handle, no allocation, no synchronization. A failed launch returns
 * OTT_ERR_HIP.
 */
ott_status_t ott_fp16_decode(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, const void* d_k, const void* d_v, int32_t max_len,
                             const int32_t* h_len, const void* d_q, void* d_out, float sm_scale,
                             void* d_work, size_t work_bytes, int32_t num_splits, void* stream);
/* ott_fp16_decode_workspace - bytes of d_work that num_splits splits need (0 for <= 1). */
size_t ott_fp16_decode_workspace(int32_t batch, int32_t num_q_heads, int32_t num_splits);

/*
 * ott_fp16_decode_noalloc - ott_fp16_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results without d_work and
 * work_bytes. The split partials go to a scratch array the library owns, one
 * copy per GPU (OTT_FP16_DECODE_SCRATCH_BYTES, held until the process ends);
 * the call allocates nothing and calls no allocating routine. The caller
 * still passes inputs and outputs.
 *   num_splits: 0 = automatic (never more than the scratch holds), 1 = no
 *   scratch used, n > 1 needs ott_fp16_decode_workspace(batch, Hq, n) <=
 *   OTT_FP16_DECODE_SCRATCH_BYTES, else OTT_ERR_SCRATCH_TOO_SMALL (nothing
 *   enqueued).
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it needs clearing: each split writes its slot before the
 * merge reads it). Calls that overlap on one GPU (other streams, other threads)
 * race on it; the caller must order them.
 */
#define OTT_FP16_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
ott_status_t ott_fp16_decode_noalloc(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, const void* d_k, const void* d_v,
                                     int32_t max_len, const int32_t* h_len, const void* d_q,
                                     void* d_out, float sm_scale, int32_t num_splits,
                                     void* stream);

/* ott_status_string - static text for a status code. */
const char* ott_status_string(ott_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* OTT_H_ */
