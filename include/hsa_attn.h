/*
 * hsa_attn.h -- hybrid long-context attention over one shared KV head
 *               (sliding window + compressed sparse + heavily compressed),
 *               hand-written HIP kernels for AMD MI355X (gfx950).
 *
 * The operations follow the hybrid attention described on the group-reading
 * wiki page "DeepSeek-V4 深度研究剖析":
 *   §5.2  SWA: the most recent n_win (= 128) raw KV tokens, attended exactly;
 *   §5.3  CSA: every m (= 4) tokens' KV pooled into one compressed entry; a
 *         lightning indexer scores the compressed blocks; a per-query top-k
 *         (512 Flash, 1024 Pro) enters the main attention;
 *   §5.4  HCA: every m' (= 128) tokens pooled into one entry, all attended;
 *   §8    KV stored in low precision (bf16 / fp8);
 *   §11.4 the heterogeneous caches: compressed KV, compressed indexer keys,
 *         raw SWA KV, and the tail of a block that is not yet complete.
 * One shared KV head (MQA): zjai.club episode 163 page, "Deep dive" §14.
 * Window and compressed entries are concatenated and share one softmax:
 * aifrontier "EP 95 解读 DeepSeek-V4 论文", section on the three components.
 *
 * Definitions used by every call (t = absolute 0-based token position):
 *   window start      s(t)  = max(0, t - n_win + 1); the window is s(t)..t.
 *   visible blocks    n_vis(t) = min(ceil(s(t)/m), floor((t+1)/m)):
 *                     complete blocks that start before the window.  This
 *                     needs m <= n_win.
 *   compression       entry[b][c] = sum_{j<m} alpha[j][c] * x[b*m+j][c],
 *                     alpha = softmax over slots j of per-slot, per-channel
 *                     logits; accumulated in float64 and rounded once to the
 *                     cache type (bf16 round-to-nearest-even, or fp8 e4m3fn
 *                     with one fp32 scale = amax/448 per 64-entry page).
 *   indexer score     I[t][b] = sum_h w[t][h] * max(0, qI[t][h] . KI_c[b]),
 *                     fp32 accumulation, no scale.
 *   top-k             the min(k, n_vis) blocks of largest score, ties to the
 *                     lower block, listed ascending, padded with -1.
 *   attention         O[t][h] = softmax_e(scale * Q[t][h] . K_e) applied to
 *                     V_e over the window rows followed by the selected (CSA)
 *                     or all visible (HCA) compressed entries: one softmax.
 *   partial RoPE      (optional; §8 keeps these channels in bf16) the last 64
 *                     channels of a key row or query head, as pairs
 *                     (d-64+2i, d-63+2i), i < 32, turn by the angle p * f_i at
 *                     position p: x' = x cos - y sin, y' = x sin + y cos, with
 *                     f_i = theta^(-2i/64) rounded to fp32; angle, cos, sin
 *                     and the turn in float64 (no fused multiply-add), then
 *                     one bf16 rounding.  A key is turned at its own position
 *                     before it is cached, so a compressed entry pools turned
 *                     keys and scores depend only on position offsets.
 *
 * Conventions
 *   - Every pointer argument that names a tensor is a DEVICE pointer unless
 *     stated otherwise; descriptor structs themselves are host memory and
 *     are read during the call only.
 *   - Layouts are row-major, innermost dimension last, as written.
 *   - bf16 tensors are passed as raw 16-bit patterns; fp8 is OCP e4m3fn.
 *   - Supported shapes: d = 128; H a multiple of 16, at most 128; indexer
 *     H_I = 4 heads of d_I = 64; page_size = 64; 1 <= m <= n_win <= 1024.
 *     Other shapes return HSA_ERR_UNSUPPORTED.
 *   - Ownership: the caller owns every buffer, including the workspace.  The
 *     library never allocates device memory and never synchronises, except in
 *     hsa_check_device_error().
 *   - Asynchrony: every compute call only enqueues work on `stream`
 *     (hsa_csa_prefill also on streams of its own, ordered with `stream` by
 *     events, so that it behaves as one call on `stream`).
 *   - Validation: arguments are checked on the host before anything is
 *     enqueued; a failed check returns a negative status, enqueues nothing,
 *     and sets a thread-local message (hsa_last_error()).
 *   - Device-side faults (a page id outside the pool, a position above the
 *     declared maximum, a cache holding fewer entries than are visible, a
 *     top-k index out of range) do not stop the call: the offending row reads
 *     as zeros, a per-device fault word is set, and hsa_check_device_error()
 *     reports it.
 *   - Workspaces: size them with the matching *_workspace_bytes() call.  A
 *     workspace needs no initialisation (every call writes whatever it later
 *     reads: no counters carry over between calls) and must not be shared by
 *     calls that may run concurrently.
 *   - Calls that run concurrently on different streams must use different
 *     workspaces and outputs.
 */
#ifndef HSA_ATTN_H
#define HSA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSA_ABI_VERSION 3

typedef enum {
  HSA_OK = 0,
  HSA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent shapes */
  HSA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (see shapes above) */
  HSA_ERR_WORKSPACE = -3,     /* ws_bytes smaller than *_workspace_bytes() */
  HSA_ERR_HIP = -4,           /* a HIP runtime call failed */
  HSA_ERR_DEVICE_FAULT = -5   /* reported by hsa_check_device_error() */
} hsa_status;

/* HSA_FP8_BF16_ROPE: the wiki's §8 KV entry, RoPE channels in BF16 and the
 * others in FP8.  A row of dim channels stores channels 0 .. dim/2-1 as
 * e4m3fn codes (dim/2 bytes, one fp32 scale per page: amax of those channels
 * over the page / 448) followed by channels dim/2 .. dim-1, the RoPE channels,
 * as bf16 (dim bytes): 3*dim/2 bytes per row.  Compressed K caches only. */
/* HSA_FP4_E2M1_MX: the wiki's §8 FP4 indexer, read as OCP MX FP4 -- e2m1
 * codes (dim/2 bytes a row, channel 2j in the low nibble of byte j) in blocks
 * of 32 channels, each block with a power-of-two scale 2^x stored as the e8m0
 * byte x + 127, x = floor(log2(amax of the block)) - 2.  The descriptor's
 * `scale` then points to the bytes [n_pages][page_size][dim/32].  Compressed
 * indexer keys only. */
typedef enum { HSA_BF16 = 0, HSA_FP8_E4M3 = 1, HSA_FP32 = 2, HSA_FP8_BF16_ROPE = 3,
               HSA_FP4_E2M1_MX = 4 } hsa_dtype;

/* Device fault bits reported by hsa_check_device_error(). */
#define HSA_FAULT_PAGE      1   /* page table entry outside [0, n_pages) */
#define HSA_FAULT_POS       2   /* a query position above max_pos */
#define HSA_FAULT_ENTRIES   4   /* n_entries[r] smaller than the visible blocks */
#define HSA_FAULT_INDEX     8   /* a top-k index outside [0, n_vis) */
#define HSA_FAULT_REQ      16   /* a listed request id outside [0, n_req) of the caches
                                   (the query reads request 0 instead) */
#define HSA_FAULT_RANGE    32   /* an attention output is not finite: a V value outside
                                   fp16's range (|v| > 65504) entered the P.V product */

/* Raw bf16 token rows of several requests.  Token p of request r lives in
 * row (p mod capacity): pass capacity >= sequence length for plain arrays
 * (prefill) or capacity = n_win for a ring (decode). */
typedef struct {
  void*   data;       /* bf16 [n_req][capacity][dim] */
  int64_t capacity;   /* rows per request, >= 1 */
  int32_t n_req;
  int32_t dim;
} hsa_tokens;

/* A paged compressed cache (compressed K, compressed V, or compressed
 * indexer keys; classical cache of §11.4).  Entry e of request r is slot
 * (e mod page_size) of physical page page_table[r*pages_per_req + e/page_size]. */
typedef struct {
  void*          data;          /* [n_pages][page_size] rows of dim dtype elements
                                   (HSA_FP8_BF16_ROPE: rows of 3*dim/2 bytes) */
  float*         scale;         /* fp8 codes: [n_pages] fp32 page scales; bf16: NULL;
                                   fp4: the e8m0 block-scale bytes (as above) */
  const int32_t* page_table;    /* [n_req][pages_per_req] physical page ids */
  int32_t*       n_entries;     /* [n_req] entries held per request */
  int32_t        n_req;
  int32_t        pages_per_req;
  int32_t        n_pages;       /* pages in the pool */
  int32_t        page_size;     /* must be 64 */
  int32_t        dim;
  int32_t        dtype;         /* hsa_dtype: bf16 or fp8 (K, V, indexer keys);
                                   HSA_FP8_BF16_ROPE (K, with an fp8 V cache);
                                   HSA_FP4_E2M1_MX (indexer keys) */
  double*        stash;         /* fp8 K / V caches that decoding appends to: float64
                                   [n_req][128][dim], the exact (pooled, unrounded)
                                   values of each request's last 128 entries, entry e
                                   at row e mod 128; NULL otherwise (see below) */
} hsa_paged;

/* Appending to an fp8 cache.  A page's scale is amax/448 over its entries,
 * so it is not final until the page is full.  The stash (part of the state
 * cache of wiki §11.4) keeps the exact values of the page still filling: every
 * append writes its entry's row and re-encodes that page from the stash with
 * the scale of the entries it now holds, so a page's codes and scale always
 * equal a from-scratch compression of exactly the entries present (the rule
 * hsa_kv_compress applies to a final partial page).  hsa_kv_compress fills
 * the stash rows of the last page it writes when the descriptor has one; 128
 * rows (two pages) let hsa_decode_rewind restore a kept page even after a
 * rejected draft started the next one. */

/* The query tokens of a call.  Either a span (req == pos == NULL): n
 * consecutive positions span_pos0 .. span_pos0+n-1 of request span_req, or a
 * list (pos non-NULL): query i is request req[i] (request i if req is NULL)
 * at position pos[i]. */
typedef struct {
  int32_t        n;
  const int32_t* req;           /* [n] or NULL */
  const int64_t* pos;           /* [n] or NULL */
  int32_t        span_req;
  int64_t        span_pos0;
  int64_t        max_pos;       /* host-known bound: every position <= max_pos */
} hsa_queries;

/* Pooling weights: alpha[j][c] = softmax over slots j of z[j][c], computed in
 * float64 (slot-order sum) and rounded once to fp32.  z, alpha: fp32 [m][dim].
 * (Compression: wiki §5.3-§5.4; softmax-weighted pooling is this library's
 * reading of "every m tokens' KV becomes one entry".) */
hsa_status hsa_pooling_weights(const float* z, int32_t m, int32_t dim, float* alpha,
                               hipStream_t stream);

/* Compress blocks [first_block, first_block + n_blocks) into request `req` of
 * `out`: block b pools tokens b*m .. b*m+m-1 of request `x_req` of x (which
 * must still hold them) with alpha [m][dim] and stores entry b (bf16, fp8
 * + page scale, or HSA_FP8_BF16_ROPE: fp8 codes of the first dim/2 channels
 * with a page scale over those channels, bf16 of the rest).  Sets
 * out->n_entries[req] = first_block + n_blocks.  Formats with page scales
 * need first_block % page_size == 0 (a page's scale is set by the call that
 * fills it from its first entry).  (Wiki §5.3, §5.4, §8.) */
hsa_status hsa_kv_compress(const hsa_tokens* x, int32_t x_req, hsa_paged* out, int32_t req,
                           int64_t first_block, int64_t n_blocks, int32_t m, const float* alpha,
                           hipStream_t stream);

/* Lightning indexer + top-k for each query (wiki §5.3; §8 for the selector).
 *   qI  bf16 [n][H_I][d_I]     w  fp32 [n][H_I]
 *   kIc paged cache of the compressed indexer keys: bf16, fp8 e4m3fn codes
 *       with one fp32 scale per 64-entry page (the low-precision indexer keys
 *       of wiki §8; key value = code value * page scale), or fp4
 *       (HSA_FP4_E2M1_MX; key value = e2m1 value * its block's 2^x)
 *   idx int32 [n][k]  out: selected blocks ascending, -1 padded
 *   score fp32 [n][k] or NULL: the indexer score of each idx entry (0 at pads)
 * Scores are computed in fp32 from bf16 operands (fp8 codes widen to bf16
 * exactly and the page scale multiplies the head sum).  Over fp4 keys the
 * indexer computes in FP4 (wiki §8): each query head is quantized to MX FP4
 * by the keys' rule (32-channel blocks, scale 2^(floor(log2 amax) - 2),
 * elements to the nearest e2m1 value, ties to even, clamped to +-6) and the
 * products of the two fp4 operands, all exact, are summed in fp32.  Listed (decode) queries
 * support up to 2^21 visible blocks per query (HSA_ERR_UNSUPPORTED beyond). */
size_t hsa_indexer_topk_workspace_bytes(const hsa_queries* q, int32_t m, int32_t n_win,
                                        int32_t k);
hsa_status hsa_indexer_topk(const hsa_queries* q, const void* qI, const float* w,
                            int32_t H_I, int32_t d_I, const hsa_paged* kIc, int32_t m,
                            int32_t n_win, int32_t k, int32_t* idx, float* score,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* The same selection over index scores rounded to bf16 (wiki §8: the index
 * scores are cast from fp32 to bf16 before the top-k selector).  Every fp32
 * score is rounded once to the nearest bf16 (ties to even) and the top-k is
 * taken over the rounded values, ties to the lower block; `score`, when not
 * NULL, receives the rounded values.  Arguments, layouts, ownership,
 * workspace (hsa_indexer_topk_workspace_bytes) and errors as
 * hsa_indexer_topk. */
hsa_status hsa_indexer_topk_bf16_scores(const hsa_queries* q, const void* qI, const float* w,
                                        int32_t H_I, int32_t d_I, const hsa_paged* kIc,
                                        int32_t m, int32_t n_win, int32_t k, int32_t* idx,
                                        float* score, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/* CSA main attention (wiki §5.2 + §5.3): per query, one softmax over the
 * window rows of win_k/win_v and the compressed entries idx[i][0..min(k,n_vis))
 * of kc/vc.  Q bf16 [n][H][d]; O [n][H][d] of o_dtype (HSA_BF16, or HSA_FP32 to
 * keep the fp32 accumulation); lse fp32 [n][H] (natural log of the softmax
 * denominator of the scaled logits) or NULL.  kc and vc: both bf16, both fp8,
 * or kc HSA_FP8_BF16_ROPE with an fp8 vc (HSA_ERR_UNSUPPORTED otherwise); a
 * mixed K row scores as (codes . q[0:d/2]) * page scale + bf16 . q[d/2:d],
 * both products exact in the fp32 accumulation. */
size_t hsa_csa_attn_workspace_bytes(const hsa_queries* q, int32_t H, int32_t n_win,
                                    int32_t k);
hsa_status hsa_csa_attn(const hsa_queries* q, const void* Q, int32_t H, int32_t d,
                        const hsa_tokens* win_k, const hsa_tokens* win_v, int32_t n_win,
                        const hsa_paged* kc, const hsa_paged* vc, int32_t m,
                        const int32_t* idx, int32_t k, float scale, void* O, int32_t o_dtype,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* A CSA layer's prefill in one call (wiki §5.3: indexer, top-k, then the
 * main attention over the selection and the window, as hsa_indexer_topk
 * followed by hsa_csa_attn).  The span is cut into stages of stage_q
 * consecutive queries (0: 16384; widened when the span would need more than
 * 1024 stages).  The selections (indexer + top-k) of even
 * and odd stages run on two streams, each with its own half of the selection
 * workspace; every stage's attention runs on a third stream, after its
 * stage's selection.  The three streams are the library's own (one set per
 * device, created on first use and kept; default priority; each with a mask
 * of every compute unit, which gives it a hardware queue of its own); events
 * order them after the work already on `stream`, and `stream` after them.
 * Results are bit-identical to the two calls on the same span.  q must be a span.  Arguments as hsa_indexer_topk (qI, w, H_I, d_I,
 * kIc, idx: required here, [n][k]) and hsa_csa_attn (Q .. lse); the indexer
 * keys are bf16, fp8 or fp4 as there, the scores fp32.  Workspace:
 * hsa_csa_prefill_workspace_bytes.  Host calls are serialised by a lock
 * (the side stream is shared); work already enqueued on `stream` before the
 * call is ordered before all of it, work enqueued after the call after all
 * of it.  Inside a stream capture the side stream joins the capture through
 * the same events. */
size_t hsa_csa_prefill_workspace_bytes(const hsa_queries* q, int32_t H, int32_t m,
                                       int32_t n_win, int32_t k);
hsa_status hsa_csa_prefill(const hsa_queries* q, const void* qI, const float* w,
                           int32_t H_I, int32_t d_I, const hsa_paged* kIc, const void* Q,
                           int32_t H, int32_t d, const hsa_tokens* win_k,
                           const hsa_tokens* win_v, int32_t n_win, const hsa_paged* kc,
                           const hsa_paged* vc, int32_t m, int32_t k, float scale,
                           int32_t* idx, void* O, int32_t o_dtype, float* lse,
                           int32_t stage_q, void* ws, size_t ws_bytes, hipStream_t stream);

/* HCA attention (wiki §5.2 + §5.4): as hsa_csa_attn with every visible
 * compressed entry (b < n_vis(t)) instead of a selection. */
size_t hsa_hca_attn_workspace_bytes(const hsa_queries* q, int32_t H, int32_t n_win,
                                    int32_t m);
hsa_status hsa_hca_attn(const hsa_queries* q, const void* Q, int32_t H, int32_t d,
                        const hsa_tokens* win_k, const hsa_tokens* win_v, int32_t n_win,
                        const hsa_paged* kc, const hsa_paged* vc, int32_t m, float scale,
                        void* O, int32_t o_dtype, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Partial RoPE over rows of bf16 heads (the definition above; wiki §8 keeps
 * the channels it turns in bf16).  x, y: bf16 [n_rows][heads][dim], dim >= 64
 * and a multiple of 8, 16-byte aligned; y == x turns in place (only the last
 * 64 channels of each head are written), otherwise y must not overlap x and
 * receives the other channels unchanged.  Row i is at position pos[i] (device
 * int64 [n_rows]) or, with pos NULL, pos0 + i.  theta > 0 and finite.
 * Prefill turns its K token rows (heads = 1) and its queries with this call
 * before compressing and attending; the decode calls turn their own.  A listed
 * position below 0 leaves its row unturned and sets HSA_FAULT_POS. */
hsa_status hsa_rope(const void* x, void* y, int64_t n_rows, int32_t heads, int32_t dim,
                    const int64_t* pos, int64_t pos0, double theta, hipStream_t stream);

typedef enum { HSA_LAYER_CSA = 0, HSA_LAYER_HCA = 1 } hsa_layer_kind;

/* One attention layer's parameters and caches for decoding a batch of B
 * requests (request b of the batch is request b of every cache). */
typedef struct {
  int32_t kind;                 /* hsa_layer_kind */
  int32_t H, d, n_win, m, topk; /* topk: CSA only */
  int32_t H_I, d_I;             /* CSA only */
  float   scale;                /* logit scale, normally 1/sqrt(d) */
  int32_t o_dtype;              /* output: HSA_BF16 or HSA_FP32 */
  const float* alpha_k;         /* [m][d]   pooling weights (hsa_pooling_weights) */
  const float* alpha_v;         /* [m][d] */
  const float* alpha_i;         /* [m][d_I] CSA only */
  hsa_tokens ring_k, ring_v;    /* raw window K/V, capacity >= n_win (state cache) */
  hsa_tokens tail_i;            /* CSA: raw indexer keys of the open block, capacity >= m */
  hsa_paged  kc, vc;            /* compressed K/V (classical cache) */
  hsa_paged  kic;               /* CSA: compressed indexer keys: bf16, or
                                   HSA_FP4_E2M1_MX (scored in FP4; the step
                                   appends MX entries; single-token steps
                                   only, no drafts) */
  double     rope_theta;        /* > 0: partial RoPE with this base (the ring
                                   and the caches then hold turned keys); 0: Q
                                   and K are used as given */
} hsa_layer;

/* One decode step of one layer for B requests (wiki §11.4 for the caches;
 * §5.2-§5.4 for the attention).  pos[b] is the position of request b's new
 * token (the request holds tokens 0..pos[b]-1).  The step
 *   1. writes the new token's K/V into ring slot pos%capacity (and KI into
 *      tail slot pos%capacity for CSA); with rope_theta > 0 the K row is
 *      turned at pos first, and the queries are turned into the workspace;
 *   2. if (pos+1) % m == 0, compresses block (pos+1)/m - 1 from the ring and
 *      tail and appends it at entry n_entries[b], which it then increments
 *      (fp8 caches: the entry's exact value goes to the stash and the page
 *      still filling is re-encoded with the scale of the entries it holds);
 *   3. runs the indexer + top-k + CSA attention, or HCA attention, for the
 *      new token's query.
 * The block completed at pos starts inside the window, so the query at pos
 * does not see it: steps 1-2 of a CSA layer ride in one of the indexer's
 * launches instead of a launch of their own, and those of an HCA layer
 * without RoPE follow the attention, in the launch that merges its splits
 * (the attention reads the new token's K/V from k_new / v_new).
 * Q bf16 [B][H][d]; k_new, v_new bf16 [B][d]; qI bf16 [B][H_I][d_I]; kI_new
 * bf16 [B][d_I]; w fp32 [B][H_I]; O [B][H][d] of L->o_dtype; lse fp32 [B][H] or NULL;
 * idx_out int32 [B][topk] or NULL (CSA).  max_pos bounds every pos[b].
 * The caller advances pos between steps.  Compressed K/V caches: bf16, or fp8
 * (HSA_FP8_E4M3, or HSA_FP8_BF16_ROPE K) with fp8 V, both with stashes.  No
 * allocation and no host synchronisation: the call can be captured in a HIP
 * graph. */
size_t hsa_decode_step_workspace_bytes(const hsa_layer* L, int32_t B, int64_t max_pos);
hsa_status hsa_decode_step(const hsa_layer* L, int32_t B, const int64_t* pos, int64_t max_pos,
                           const void* Q, const void* k_new, const void* v_new,
                           const void* qI, const void* kI_new, const float* w,
                           void* O, float* lse, int32_t* idx_out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as hsa_decode_step, arguments and results alike, with its workspace
 * taken from the library's own device scratch of HSA_NOALLOC_SCRATCH_BYTES
 * (one copy per GPU, held until the process ends) instead of a caller buffer.
 * A step whose hsa_decode_step_workspace_bytes() exceeds it returns
 * HSA_ERR_WORKSPACE and enqueues nothing (128 MiB covers 16 requests at 1M
 * tokens).  The call allocates nothing and does not synchronise.  Every call
 * on one GPU shares that GPU's scratch (the step needs it cleared of nothing:
 * it writes whatever it later reads), so calls that may overlap on one GPU
 * -- on different streams, or from different threads -- race; serialise them
 * or use hsa_decode_step with workspaces of their own. */
#define HSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
hsa_status hsa_decode_step_noalloc(const hsa_layer* L, int32_t B, const int64_t* pos,
                                   int64_t max_pos, const void* Q, const void* k_new,
                                   const void* v_new, const void* qI, const void* kI_new,
                                   const float* w, void* O, float* lse, int32_t* idx_out,
                                   hipStream_t stream);

/* A draft of n_tok tokens per request for speculative decoding (the draft's
 * queries are verified together; wiki §11.4 for the caches kept in sync).
 * Tokens pos[b] .. pos[b]+n_tok-1 of request b are appended in order, as
 * n_tok single-token steps would append them (rings, tail, every block they
 * complete), then query i of request b, at position pos[b]+i, runs the
 * indexer + top-k + CSA attention or the HCA attention and sees exactly what a
 * single-token step at that position sees: a block completed later in the
 * draft is not visible to it, and its window rows survive because the rings
 * must hold n_win + n_tok - 1 tokens.  Arrays are [B][n_tok][...] versions of
 * hsa_decode_step's (row b * n_tok + i is token / query i of request b): Q
 * [B][n_tok][H][d]; k_new, v_new [B][n_tok][d]; qI [B][n_tok][H_I][d_I];
 * kI_new [B][n_tok][d_I]; w [B][n_tok][H_I]; O [B][n_tok][H][d]; lse
 * [B][n_tok][H] or NULL; idx_out [B][n_tok][topk] or NULL.  1 <= n_tok <= 256;
 * max_pos bounds every pos[b] + n_tok - 1.  A CSA layer's indexer tail must
 * hold m + n_tok - 1 rows, so that hsa_decode_rewind can drop any rejected
 * suffix.  The caller advances pos by the accepted tokens and rewinds the
 * caches to them with hsa_decode_rewind (the draft appended every token).
 * No allocation and no host synchronisation. */
size_t hsa_decode_draft_workspace_bytes(const hsa_layer* L, int32_t B, int32_t n_tok,
                                        int64_t max_pos);
hsa_status hsa_decode_draft(const hsa_layer* L, int32_t B, int32_t n_tok, const int64_t* pos,
                            int64_t max_pos, const void* Q, const void* k_new, const void* v_new,
                            const void* qI, const void* kI_new, const float* w, void* O,
                            float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Rewind a layer's caches after a draft whose suffix was rejected (zjai.club
 * episode 163 page, "Deep dive" §16: the caches stay in step across prefill,
 * decode and speculative decode).  Request b keeps tokens 0 .. keep[b]-1:
 * n_entries[b] of the compressed K, V (and, CSA, indexer-key) caches becomes
 * keep[b] / m, dropping every block a rejected token completed.  The rings
 * and the indexer tail need no change: a slot is position mod capacity, so
 * the next tokens overwrite the rejected rows before any query reads them,
 * and the sizes hsa_decode_draft requires keep the kept rows intact.
 * keep int64 [B] (device).  bf16 caches only.  A keep[b] < 0, or one asking
 * for more blocks than a cache holds, leaves request b unchanged and raises
 * HSA_FAULT_POS / HSA_FAULT_ENTRIES.  No allocation, no host synchronisation. */
hsa_status hsa_decode_rewind(const hsa_layer* L, int32_t B, const int64_t* keep,
                             hipStream_t stream);

/* Optional kernel timing (tracing).  While enabled for a kernel, every launch
 * of it is timed with a pair of HIP events on its stream; read returns the
 * summed elapsed milliseconds and the number of launches since the previous
 * read (synchronising on the events).  Single kernels (SCAN, GEMM, ATTN) hand
 * the pair to their own dispatch (hipExtLaunchKernelGGL), so the time is the
 * kernel's execution alone; SEL and COMPRESS bracket their launch sequence
 * with recorded events.  For eager execution only: do not enable it while
 * capturing a graph. */
#define HSA_K_INDEXER_SCAN  0   /* decode: score scan + first histogram (one kernel) */
#define HSA_K_INDEXER_GEMM  1   /* prefill: MFMA score GEMM (one kernel per query chunk) */
#define HSA_K_INDEXER_SEL   2   /* histogram / select / refine / emit (several kernels) */
#define HSA_K_ATTN          3   /* gather + online-softmax attention (one kernel; no merge) */
#define HSA_K_COMPRESS      4   /* block pooling */
#define HSA_K_COUNT         5
hsa_status hsa_kernel_timing(int32_t kernel_id, int32_t enable);
hsa_status hsa_kernel_timing_read(int32_t kernel_id, double* total_ms, int64_t* launches);

/* Helpers. */
const char* hsa_status_string(hsa_status s);
const char* hsa_last_error(void);                 /* thread-local detail of the last failure */
hsa_status  hsa_check_device_error(hipStream_t stream, int32_t* fault_bits);
                                                  /* synchronises `stream`, reads and clears
                                                     the current device's fault word */
int32_t     hsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HSA_ATTN_H */
