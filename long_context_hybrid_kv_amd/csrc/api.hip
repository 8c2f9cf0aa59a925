// C ABI of libhsa_attn: argument validation, workspace sizing, dispatch to the
// gfx950 kernels, status strings and the per-device fault word.
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "update.h"

namespace hsa {

// Device fault word: kernels OR HSA_FAULT_* bits into it (one copy per device).
__device__ int g_fault_word;

int* fault_word() {
  static std::mutex mu;
  static int* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_fault_word)) != hipSuccess) return nullptr;
    ptrs[dev] = (int*)p;
  }
  return ptrs[dev];
}

// ---------------------------------------------------------------- allocation-free decode

// Workspace of hsa_decode_step_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: host code uses only the address that
// hipGetSymbolAddress returns for the current device (scratch_ptr()).
static __device__ __align__(256) uint8_t scratch[HSA_NOALLOC_SCRATCH_BYTES];

static void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// ---------------------------------------------------------------- kernel timing

struct TimerState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  size_t used = 0;
};
static TimerState g_timers[HSA_K_COUNT];
static std::mutex g_timer_mu;

KernelTimer::KernelTimer(int id, hipStream_t s, bool ext)
    : id_(id), s_(s), slot_(nullptr), ext_(ext) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerState& t = g_timers[id];
  if (!t.on) return;
  if (t.used == t.ev.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
    t.ev.emplace_back(a, b);
  }
  auto* pr = &t.ev[t.used++];
  slot_ = pr;
  if (!ext_) (void)hipEventRecord(pr->first, s);
}

KernelTimer::~KernelTimer() {
  if (slot_ && !ext_) (void)hipEventRecord(((std::pair<hipEvent_t, hipEvent_t>*)slot_)->second, s_);
}

hipEvent_t KernelTimer::start() const {
  return ((std::pair<hipEvent_t, hipEvent_t>*)slot_)->first;
}

hipEvent_t KernelTimer::stop() const {
  return ((std::pair<hipEvent_t, hipEvent_t>*)slot_)->second;
}

static thread_local std::string g_err;

static hsa_status fail(hsa_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define REQ(cond, msg) \
  do { if (!(cond)) return fail(HSA_ERR_INVALID_ARG, msg); } while (0)
#define SUP(cond, msg) \
  do { if (!(cond)) return fail(HSA_ERR_UNSUPPORTED, msg); } while (0)

static hsa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return HSA_OK;
  return fail(HSA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

static int64_t nvis_host(int64_t t, int m, int n_win) {
  int64_t s = t - n_win + 1 < 0 ? 0 : t - n_win + 1;
  int64_t a = (s + m - 1) / m, b = (t + 1) / m;
  return a < b ? a : b;
}

// allow_mixed: the cache may be HSA_FP8_BF16_ROPE (compressed K, dim 128);
// allow_fp4: HSA_FP4_E2M1_MX (compressed indexer keys, dim 64)
static hsa_status check_paged(const hsa_paged* p, const char* name, int dim, bool allow_fp8,
                              bool allow_mixed = false, bool allow_fp4 = false) {
  std::string n(name);
  REQ(p, n + ": null descriptor");
  REQ(p->data && p->page_table && p->n_entries, n + ": null data, page_table or n_entries");
  REQ(p->n_req >= 1 && p->pages_per_req >= 1 && p->n_pages >= 1, n + ": empty cache");
  SUP(p->page_size == kPage, n + ": page_size must be 64");
  SUP(p->dim == dim, n + ": unsupported dim");
  REQ(p->dtype == HSA_BF16 || p->dtype == HSA_FP8_E4M3 || p->dtype == HSA_FP8_BF16_ROPE ||
          p->dtype == HSA_FP4_E2M1_MX,
      n + ": unknown dtype");
  SUP(allow_fp8 || p->dtype == HSA_BF16 || (allow_fp4 && p->dtype == HSA_FP4_E2M1_MX),
      n + (allow_fp4 ? ": must be bf16 or fp4" : ": must be bf16"));
  SUP(p->dtype != HSA_FP8_BF16_ROPE || (allow_mixed && p->dim == kD),
      n + ": the mixed bf16-RoPE / fp8 format is for compressed K caches of dim 128");
  SUP(p->dtype != HSA_FP4_E2M1_MX || (allow_fp4 && p->dim == kDI),
      n + ": fp4 is for compressed indexer keys of dim 64");
  REQ(p->dtype == HSA_BF16 || p->scale, n + ": fp8 cache needs page scales");
  SUP(p->n_pages < (1 << 25), n + ": pool rows must be addressable by a 32-bit row id");
  return HSA_OK;
}

static hsa_status check_tokens(const hsa_tokens* t, const char* name, int dim, int64_t need_cap) {
  std::string n(name);
  REQ(t && t->data, n + ": null");
  REQ(t->n_req >= 1 && t->capacity >= 1, n + ": empty");
  SUP(t->dim == dim, n + ": unsupported dim");
  REQ(t->capacity >= need_cap, n + ": capacity smaller than the rows it must hold");
  SUP(t->capacity * t->n_req < (int64_t(1) << 31) - 2, n + ": rows must be addressable by a 32-bit row id");
  return HSA_OK;
}

static hsa_status check_queries(const hsa_queries* q, int n_req) {
  REQ(q, "queries: null");
  REQ(q->n >= 1, "queries: n must be >= 1");
  REQ(q->max_pos >= 0 && q->max_pos < (int64_t(1) << 40), "queries: bad max_pos");
  if (!q->pos) {
    REQ(!q->req, "queries: req given without pos");
    REQ(q->span_req >= 0 && q->span_req < n_req, "queries: span_req out of range");
    REQ(q->span_pos0 >= 0 && q->span_pos0 + q->n - 1 <= q->max_pos,
        "queries: span exceeds max_pos");
  } else {
    REQ(q->req || q->n <= n_req, "queries: implicit request ids exceed the caches");
  }
  return HSA_OK;
}

static bool is_span(const hsa_queries* q) { return !q->pos; }

static hsa_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return HSA_OK;
  if (!ws || have < need)
    return fail(HSA_ERR_WORKSPACE, "workspace: " + std::to_string(have) + " bytes given, " +
                                       std::to_string(need) + " needed");
  return HSA_OK;
}

static size_t csa_entries(int n_win, int k) { return (size_t)n_win + k; }

static hsa_status check_attn_common(const hsa_queries* q, const void* Q, int H, int d,
                                    const hsa_tokens* wk, const hsa_tokens* wv, int n_win,
                                    const hsa_paged* kc, const hsa_paged* vc, int m, float scale,
                                    void* O) {
  REQ(kc && vc, "attention: null cache");
  REQ(scale > 0.f && scale < INFINITY, "attention: scale must be positive and finite");
  hsa_status s;
  if ((s = check_paged(kc, "kc", kD, true, true)) != HSA_OK) return s;
  if ((s = check_paged(vc, "vc", kD, true)) != HSA_OK) return s;
  if ((s = check_queries(q, kc->n_req)) != HSA_OK) return s;
  REQ(kc->n_req == vc->n_req, "attention: kc and vc differ in n_req");
  SUP(kc->dtype == vc->dtype || (kc->dtype == HSA_FP8_BF16_ROPE && vc->dtype == HSA_FP8_E4M3),
      "attention: kc and vc must both be bf16 or both fp8 (or a mixed kc with an fp8 vc)");
  REQ(Q && O, "attention: null Q or O");
  SUP(d == kD, "attention: d must be 128");
  SUP(H >= 16 && H <= 128 && H % 16 == 0, "attention: H must be a multiple of 16 in [16, 128]");
  REQ(n_win >= 1 && m >= 1, "attention: n_win and m must be >= 1");
  SUP(m <= n_win, "attention: m > n_win leaves tokens uncovered");
  int64_t need_cap = q->max_pos + 1 < n_win ? q->max_pos + 1 : n_win;
  if ((s = check_tokens(wk, "win_k", kD, need_cap)) != HSA_OK) return s;
  if ((s = check_tokens(wv, "win_v", kD, need_cap)) != HSA_OK) return s;
  REQ(wk->n_req >= kc->n_req && wv->n_req >= kc->n_req, "attention: window holds fewer requests");
  int64_t nv = nvis_host(q->max_pos, m, n_win);
  REQ((int64_t)kc->pages_per_req * kPage >= nv && (int64_t)vc->pages_per_req * kPage >= nv,
      "attention: page table shorter than the visible blocks");
  return HSA_OK;
}

}  // namespace hsa

using namespace hsa;

extern "C" {

int32_t hsa_abi_version(void) { return HSA_ABI_VERSION; }

hsa_status hsa_kernel_timing(int32_t kernel_id, int32_t enable) {
  REQ(kernel_id >= 0 && kernel_id < HSA_K_COUNT, "kernel_timing: unknown kernel id");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timers[kernel_id].on = enable != 0;
  return HSA_OK;
}

hsa_status hsa_kernel_timing_read(int32_t kernel_id, double* total_ms, int64_t* launches) {
  REQ(kernel_id >= 0 && kernel_id < HSA_K_COUNT, "kernel_timing_read: unknown kernel id");
  REQ(total_ms && launches, "kernel_timing_read: null output");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerState& t = g_timers[kernel_id];
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    hipError_t e = hipEventSynchronize(t.ev[i].second);
    if (e != hipSuccess) return hip_status(e, "hipEventSynchronize");
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, t.ev[i].first, t.ev[i].second)) != hipSuccess)
      return hip_status(e, "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)t.used;
  t.used = 0;
  return HSA_OK;
}

const char* hsa_last_error(void) { return g_err.c_str(); }

const char* hsa_status_string(hsa_status s) {
  switch (s) {
    case HSA_OK: return "ok";
    case HSA_ERR_INVALID_ARG: return "invalid argument";
    case HSA_ERR_UNSUPPORTED: return "unsupported";
    case HSA_ERR_WORKSPACE: return "workspace too small";
    case HSA_ERR_HIP: return "HIP runtime error";
    case HSA_ERR_DEVICE_FAULT: return "device fault";
  }
  return "unknown status";
}

hsa_status hsa_check_device_error(hipStream_t stream, int32_t* fault_bits) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "hipStreamSynchronize");
  int* p = fault_word();
  if (!p) return fail(HSA_ERR_HIP, "fault word unavailable");
  int v = 0;
  if ((e = hipMemcpy(&v, p, sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_status(e, "hipMemcpy");
  if (v) {
    int zero = 0;
    if ((e = hipMemcpy(p, &zero, sizeof(int), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_status(e, "hipMemcpy");
  }
  if (fault_bits) *fault_bits = v;
  return v ? fail(HSA_ERR_DEVICE_FAULT, "device fault bits " + std::to_string(v)) : HSA_OK;
}

hsa_status hsa_pooling_weights(const float* z, int32_t m, int32_t dim, float* alpha,
                               hipStream_t stream) {
  REQ(z && alpha, "pooling_weights: null pointer");
  REQ(m >= 1 && m <= 4096 && dim >= 1 && dim <= 4096, "pooling_weights: bad m or dim");
  return hip_status(launch_pooling_weights(z, m, dim, alpha, stream), "pooling_weights");
}

hsa_status hsa_kv_compress(const hsa_tokens* x, int32_t x_req, hsa_paged* out, int32_t req,
                           int64_t first_block, int64_t n_blocks, int32_t m, const float* alpha,
                           hipStream_t stream) {
  REQ(out, "kv_compress: null output");
  SUP(out->dim == kD || out->dim == kDI, "kv_compress: dim must be 128 or 64");
  hsa_status s;
  if ((s = check_paged(out, "out", out->dim, true, true, true)) != HSA_OK) return s;
  if ((s = check_tokens(x, "x", out->dim, 1)) != HSA_OK) return s;
  REQ(alpha, "kv_compress: null alpha");
  REQ(m >= 1 && m <= 4096, "kv_compress: bad m");
  REQ(x->capacity >= m, "kv_compress: x holds fewer than m rows");
  REQ(req >= 0 && req < out->n_req, "kv_compress: req out of range");
  REQ(x_req >= 0 && x_req < x->n_req, "kv_compress: x_req out of range");
  REQ(first_block >= 0 && n_blocks >= 0, "kv_compress: negative range");
  REQ(first_block + n_blocks <= (int64_t)out->pages_per_req * kPage,
      "kv_compress: range exceeds the request's pages");
  REQ(out->dtype == HSA_BF16 || first_block % kPage == 0,
      "kv_compress: fp8 ranges must start on a page boundary");
  return hip_status(launch_compress(*x, x_req, *out, req, first_block, n_blocks, m, alpha, stream),
                    "kv_compress");
}

hsa_status hsa_rope(const void* x, void* y, int64_t n_rows, int32_t heads, int32_t dim,
                    const int64_t* pos, int64_t pos0, double theta, hipStream_t stream) {
  REQ(n_rows >= 0, "rope: negative n_rows");
  REQ(heads >= 1 && heads <= 4096, "rope: heads must be in [1, 4096]");
  REQ(dim >= kRopeDim && dim % 8 == 0 && dim <= 4096,
      "rope: dim must be a multiple of 8 in [64, 4096]");
  REQ(std::isfinite(theta) && theta > 0.0, "rope: theta must be finite and > 0");
  if (n_rows == 0) return HSA_OK;
  REQ(x && y, "rope: null x or y");
  REQ((((uintptr_t)x | (uintptr_t)y) & 15) == 0, "rope: x and y must be 16-byte aligned");
  REQ(pos || (pos0 >= 0 && pos0 <= INT64_MAX - n_rows), "rope: positions out of range");
  const uintptr_t bytes = (uintptr_t)n_rows * heads * dim * sizeof(uint16_t);
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
  REQ(xa == ya || xa + bytes <= ya || ya + bytes <= xa, "rope: y overlaps x without equalling it");
  return hip_status(launch_rope(x, y, n_rows, heads, dim, pos, pos0, theta, stream), "rope");
}

size_t hsa_indexer_topk_workspace_bytes(const hsa_queries* q, int32_t m, int32_t n_win,
                                        int32_t k) {
  if (!q || q->n < 1 || m < 1 || n_win < 1 || k < 1 || q->max_pos < 0) return 0;
  return indexer_ws_bytes(q->n, nvis_host(q->max_pos, m, n_win), k, is_span(q), 1);
}

static hsa_status indexer_topk(const hsa_queries* q, const void* qI, const float* w, int32_t H_I,
                               int32_t d_I, const hsa_paged* kIc, int32_t m, int32_t n_win,
                               int32_t k, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                               hipStream_t stream, bool s16) {
  hsa_status s;
  if ((s = check_paged(kIc, "kIc", kDI, true, false, true)) != HSA_OK) return s;
  if ((s = check_queries(q, kIc->n_req)) != HSA_OK) return s;
  REQ(qI && w && idx, "indexer_topk: null qI, w or idx");
  SUP(H_I == kHI && d_I == kDI, "indexer_topk: H_I must be 4 and d_I 64");
  REQ(m >= 1 && n_win >= 1, "indexer_topk: bad m or n_win");
  SUP(m <= n_win, "indexer_topk: m > n_win leaves tokens uncovered");
  REQ(k >= 1 && k <= (1 << 20), "indexer_topk: k out of range");
  int64_t nv = nvis_host(q->max_pos, m, n_win);
  REQ((int64_t)kIc->pages_per_req * kPage >= nv, "indexer_topk: page table too short");
  SUP(is_span(q) || nv <= indexer_max_blocks(),
      "indexer_topk: decode rows longer than 2^21 visible blocks are not supported");
  if ((s = check_ws(ws, ws_bytes, hsa_indexer_topk_workspace_bytes(q, m, n_win, k))) != HSA_OK)
    return s;
  return hip_status(launch_indexer(*q, qI, w, *kIc, m, n_win, k, idx, score, ws, ws_bytes, stream,
                                   nullptr, 1, s16),
                    "indexer_topk");
}

hsa_status hsa_indexer_topk(const hsa_queries* q, const void* qI, const float* w, int32_t H_I,
                            int32_t d_I, const hsa_paged* kIc, int32_t m, int32_t n_win,
                            int32_t k, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return indexer_topk(q, qI, w, H_I, d_I, kIc, m, n_win, k, idx, score, ws, ws_bytes, stream,
                      false);
}

hsa_status hsa_indexer_topk_bf16_scores(const hsa_queries* q, const void* qI, const float* w,
                                        int32_t H_I, int32_t d_I, const hsa_paged* kIc, int32_t m,
                                        int32_t n_win, int32_t k, int32_t* idx, float* score,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  return indexer_topk(q, qI, w, H_I, d_I, kIc, m, n_win, k, idx, score, ws, ws_bytes, stream,
                      true);
}

size_t hsa_csa_attn_workspace_bytes(const hsa_queries* q, int32_t H, int32_t n_win, int32_t k) {
  if (!q || q->n < 1 || H < 16 || n_win < 1 || k < 1) return 0;
  return attn_ws_bytes(q->n, H, (int64_t)csa_entries(n_win, k), is_span(q),
                       attn_decode_cps(k, n_win));
}

hsa_status hsa_csa_attn(const hsa_queries* q, const void* Q, int32_t H, int32_t d,
                        const hsa_tokens* win_k, const hsa_tokens* win_v, int32_t n_win,
                        const hsa_paged* kc, const hsa_paged* vc, int32_t m, const int32_t* idx,
                        int32_t k, float scale, void* O, int32_t o_dtype, float* lse, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  hsa_status s;
  REQ(o_dtype == HSA_BF16 || o_dtype == HSA_FP32, "csa_attn: o_dtype must be bf16 or fp32");
  if ((s = check_attn_common(q, Q, H, d, win_k, win_v, n_win, kc, vc, m, scale, O)) != HSA_OK)
    return s;
  REQ(idx, "csa_attn: null idx");
  REQ(k >= 1 && k <= (1 << 20), "csa_attn: k out of range");
  if ((s = check_ws(ws, ws_bytes, hsa_csa_attn_workspace_bytes(q, H, n_win, k))) != HSA_OK)
    return s;
  return hip_status(launch_attn(*q, Q, H, *win_k, *win_v, n_win, *kc, *vc, m, idx, k, scale, O,
                                o_dtype, lse, ws, ws_bytes, stream),
                    "csa_attn");
}

// ---------------------------------------------------------------- CSA prefill, pipelined

// The streams of the pipeline -- sel[0], sel[1]: the selections of even and
// odd stages, att: every stage's attention -- and the events that order them,
// one set per device, created on first use and kept until the process ends.
// The caller's stream only forks the pipeline and waits for it.
struct PipeState {
  hipStream_t sel[2] = {nullptr, nullptr}, att = nullptr;
  std::vector<hipEvent_t> ev;
};
static std::mutex g_pipe_mu;
static PipeState g_pipe[64];
constexpr int kStageQueries = 16384;
constexpr int kMaxStages = 1024;

// one selection workspace per selection stream
static size_t csa_prefill_sel_bytes(const hsa_queries* q, int m, int n_win, int k) {
  return (hsa_indexer_topk_workspace_bytes(q, m, n_win, k) + 255) & ~size_t(255);
}

size_t hsa_csa_prefill_workspace_bytes(const hsa_queries* q, int32_t H, int32_t m, int32_t n_win,
                                       int32_t k) {
  if (!q || q->pos || H < 16) return 0;
  // every stage's selection fits the full span's layout (the score rows are
  // as long as the longest row of the span, the passes as wide); span
  // attention needs none
  return 2 * csa_prefill_sel_bytes(q, m, n_win, k) + hsa_csa_attn_workspace_bytes(q, H, n_win, k);
}

hsa_status hsa_csa_prefill(const hsa_queries* q, const void* qI, const float* w, int32_t H_I,
                           int32_t d_I, const hsa_paged* kIc, const void* Q, int32_t H, int32_t d,
                           const hsa_tokens* win_k, const hsa_tokens* win_v, int32_t n_win,
                           const hsa_paged* kc, const hsa_paged* vc, int32_t m, int32_t k,
                           float scale, int32_t* idx, void* O, int32_t o_dtype, float* lse,
                           int32_t stage_q, void* ws, size_t ws_bytes, hipStream_t stream) {
  hsa_status s;
  REQ(q, "csa_prefill: null queries");
  REQ(!q->pos && !q->req, "csa_prefill: queries must be a span");
  REQ(stage_q >= 0, "csa_prefill: negative stage size");
  REQ(o_dtype == HSA_BF16 || o_dtype == HSA_FP32, "csa_prefill: o_dtype must be bf16 or fp32");
  if ((s = check_paged(kIc, "kIc", kDI, true, false, true)) != HSA_OK) return s;
  if ((s = check_attn_common(q, Q, H, d, win_k, win_v, n_win, kc, vc, m, scale, O)) != HSA_OK)
    return s;
  REQ(kIc->n_req == kc->n_req, "csa_prefill: kIc and kc differ in n_req");
  REQ(qI && w && idx, "csa_prefill: null qI, w or idx");
  SUP(H_I == kHI && d_I == kDI, "csa_prefill: H_I must be 4 and d_I 64");
  REQ(k >= 1 && k <= (1 << 20), "csa_prefill: k out of range");
  REQ((int64_t)kIc->pages_per_req * kPage >= nvis_host(q->max_pos, m, n_win),
      "csa_prefill: indexer page table too short");
  if ((s = check_ws(ws, ws_bytes, hsa_csa_prefill_workspace_bytes(q, H, m, n_win, k))) != HSA_OK)
    return s;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(HSA_ERR_HIP, "csa_prefill: no current device");
  // at most kMaxStages stages (one event each): a smaller stage_q is widened
  int S = stage_q > 0 ? stage_q : kStageQueries;
  if ((q->n + (int64_t)S - 1) / S > kMaxStages) S = (int)((q->n + kMaxStages - 1) / kMaxStages);
  const int n_st = (int)((q->n + (int64_t)S - 1) / S);
  std::lock_guard<std::mutex> lk(g_pipe_mu);
  PipeState& P = g_pipe[dev];
  if (!P.sel[0] || !P.sel[1] || !P.att) {
    // a mask of every compute unit: no CU is left out, and a stream with a CU
    // mask gets a hardware queue of its own instead of sharing one of the
    // process's few queues round-robin with other streams, which would
    // serialise the stages (measured: 12.1 ms for the 128K CSA layer, 12.6 ms
    // when three streams were created before it).  Such streams synchronise
    // with the legacy default stream, which is why no stage runs on the
    // caller's stream.
    int n_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e, "csa_prefill: CU count");
    std::vector<uint32_t> mask((size_t)(n_cu + 31) / 32, 0u);
    for (int i = 0; i < n_cu; ++i) mask[i / 32] |= 1u << (i % 32);
    for (hipStream_t* st : {&P.sel[0], &P.sel[1], &P.att}) {
      if (*st) continue;
      e = hipExtStreamCreateWithCUMask(st, (uint32_t)mask.size(), mask.data());
      if (e != hipSuccess) return hip_status(e, "csa_prefill: stream");
    }
  }
  // events: [0] fork, [1 + p] stage p's selection done, [1 + n_st ..] joins
  while ((int)P.ev.size() < n_st + 4) {
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_status(e, "csa_prefill: event");
    P.ev.push_back(ev);
  }
  const size_t o_row = (size_t)H * kD * (o_dtype == HSA_FP32 ? 4 : 2);
  const size_t half = csa_prefill_sel_bytes(q, m, n_win, k);
  // the pipeline's streams start after everything already enqueued on `stream`
  hipError_t e = hipEventRecord(P.ev[0], stream);
  for (hipStream_t st : {P.sel[0], P.sel[1], P.att})
    if (e == hipSuccess) e = hipStreamWaitEvent(st, P.ev[0], 0);
  for (int p = 0; p < n_st && e == hipSuccess; ++p) {
    const int64_t c0 = (int64_t)p * S;
    const int nq = (int)(q->n - c0 < S ? q->n - c0 : S);
    hsa_queries sub = *q;
    sub.n = nq;
    sub.span_pos0 = q->span_pos0 + c0;
    sub.max_pos = sub.span_pos0 + nq - 1;
    int32_t* idx_p = idx + c0 * k;
    // consecutive stages' selections on two streams, each with its own half of
    // the workspace (a stream's stages reuse its half in order)
    hipStream_t ss = P.sel[p & 1];
    e = launch_indexer(sub, (const u16*)qI + c0 * kHI * kDI, w + c0 * kHI, *kIc, m, n_win, k,
                       idx_p, nullptr, (uint8_t*)ws + (p & 1) * half, half, ss, nullptr, 1,
                       false);
    if (e == hipSuccess) e = hipEventRecord(P.ev[1 + p], ss);
    if (e == hipSuccess) e = hipStreamWaitEvent(P.att, P.ev[1 + p], 0);
    if (e == hipSuccess)
      e = launch_attn(sub, (const u16*)Q + c0 * H * kD, H, *win_k, *win_v, n_win, *kc, *vc, m,
                      idx_p, k, scale, (uint8_t*)O + c0 * o_row, o_dtype,
                      lse ? lse + c0 * H : nullptr, nullptr, 0, P.att);
  }
  // `stream` waits for the three streams, also after a failed launch
  hipError_t j = hipSuccess;
  int ji = 1 + n_st;
  for (hipStream_t st : {P.sel[0], P.sel[1], P.att}) {
    if (j == hipSuccess) j = hipEventRecord(P.ev[ji], st);
    if (j == hipSuccess) j = hipStreamWaitEvent(stream, P.ev[ji], 0);
    ++ji;
  }
  if (e != hipSuccess) return hip_status(e, "csa_prefill");
  return hip_status(j, "csa_prefill: join");
}

size_t hsa_hca_attn_workspace_bytes(const hsa_queries* q, int32_t H, int32_t n_win, int32_t m) {
  if (!q || q->n < 1 || H < 16 || n_win < 1 || m < 1 || q->max_pos < 0) return 0;
  return attn_ws_bytes(q->n, H, n_win + nvis_host(q->max_pos, m, n_win), is_span(q),
                       attn_decode_cps(0, n_win));
}

hsa_status hsa_hca_attn(const hsa_queries* q, const void* Q, int32_t H, int32_t d,
                        const hsa_tokens* win_k, const hsa_tokens* win_v, int32_t n_win,
                        const hsa_paged* kc, const hsa_paged* vc, int32_t m, float scale, void* O,
                        int32_t o_dtype, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  hsa_status s;
  REQ(o_dtype == HSA_BF16 || o_dtype == HSA_FP32, "hca_attn: o_dtype must be bf16 or fp32");
  if ((s = check_attn_common(q, Q, H, d, win_k, win_v, n_win, kc, vc, m, scale, O)) != HSA_OK)
    return s;
  if ((s = check_ws(ws, ws_bytes, hsa_hca_attn_workspace_bytes(q, H, n_win, m))) != HSA_OK)
    return s;
  return hip_status(launch_attn(*q, Q, H, *win_k, *win_v, n_win, *kc, *vc, m, nullptr, 0, scale,
                                O, o_dtype, lse, ws, ws_bytes, stream),
                    "hca_attn");
}

// The compressed K / V caches a decode step, draft or rewind may append to:
// both bf16, or fp8 (a mixed K with an fp8 V, or both fp8) with a stash each.
static hsa_status check_append_caches(const hsa_layer* L, const std::string& who) {
  const int kt = L->kc.dtype, vt = L->vc.dtype;
  const bool bf = kt == HSA_BF16 && vt == HSA_BF16;
  const bool f8 = (kt == HSA_FP8_E4M3 || kt == HSA_FP8_BF16_ROPE) && vt == HSA_FP8_E4M3;
  SUP(bf || f8, who + ": K / V caches must be both bf16, or fp8 (K fp8 or mixed, V fp8)");
  REQ(bf || (L->kc.stash && L->vc.stash),
      who + ": appending to fp8 caches needs their stashes (the exact values of the open page)");
  return HSA_OK;
}

// decode_step workspace: [indexer][selected ids][attention], 256-byte aligned
static size_t rnd256(size_t b) { return (b + 255) & ~size_t(255); }

static size_t rope_q_bytes(const hsa_layer* L, size_t n_q) {
  return L->rope_theta > 0.0 ? rnd256(sizeof(uint16_t) * n_q * L->H * kD) : 0;
}

// (with RoPE the turned queries follow the attention's part)
static void decode_parts(const hsa_layer* L, int32_t B, int64_t max_pos, size_t* p_idx,
                         size_t* p_sel, size_t* p_attn) {
  hsa_queries q{};
  q.n = B;
  q.pos = (const int64_t*)1;   // list mode for sizing only
  q.max_pos = max_pos;
  *p_idx = *p_sel = 0;
  if (L->kind == HSA_LAYER_CSA) {
    *p_idx = rnd256(hsa_indexer_topk_workspace_bytes(&q, L->m, L->n_win, L->topk));
    *p_sel = rnd256(sizeof(int32_t) * (size_t)B * L->topk);
    *p_attn = rnd256(hsa_csa_attn_workspace_bytes(&q, L->H, L->n_win, L->topk));
  } else {
    *p_attn = rnd256(hsa_hca_attn_workspace_bytes(&q, L->H, L->n_win, L->m));
  }
}

size_t hsa_decode_step_workspace_bytes(const hsa_layer* L, int32_t B, int64_t max_pos) {
  if (!L || B < 1 || max_pos < 0 || L->m < 1 || L->n_win < 1 || L->H < 16) return 0;
  if (L->kind == HSA_LAYER_CSA && L->topk < 1) return 0;
  size_t a, b, c;
  decode_parts(L, B, max_pos, &a, &b, &c);
  return a + b + c + rope_q_bytes(L, (size_t)B);
}

// Validation shared by the single-token step and the draft (n_tok tokens per
// request; the rings must keep the first draft query's window while the
// draft's later tokens are written).
static hsa_status check_decode(const hsa_layer* L, int32_t B, int32_t n_tok, const int64_t* pos,
                               int64_t max_pos, const void* Q, const void* k_new,
                               const void* v_new, const void* qI, const void* kI_new,
                               const float* w, void* O) {
  REQ(L, "decode: null layer");
  REQ(L->kind == HSA_LAYER_CSA || L->kind == HSA_LAYER_HCA, "decode: unknown layer kind");
  REQ(B >= 1 && pos && Q && k_new && v_new && O, "decode: null argument or B < 1");
  REQ(n_tok >= 1 && n_tok <= 256, "decode: n_tok must be in [1, 256]");
  REQ(L->alpha_k && L->alpha_v, "decode: null pooling weights");
  REQ(L->o_dtype == HSA_BF16 || L->o_dtype == HSA_FP32, "decode: o_dtype must be bf16 or fp32");
  REQ(std::isfinite(L->rope_theta) && L->rope_theta >= 0.0,
      "decode: rope_theta must be finite and >= 0 (0: no RoPE)");
  {
    hsa_status sa = check_append_caches(L, "decode");
    if (sa != HSA_OK) return sa;
  }
  REQ(L->kc.n_req >= B && L->vc.n_req >= B && L->ring_k.n_req >= B && L->ring_v.n_req >= B,
      "decode: caches hold fewer than B requests");
  REQ(L->n_win >= 1 && L->m >= 1 && L->m <= L->n_win, "decode: need 1 <= m <= n_win");
  hsa_queries q{};
  q.n = B * n_tok;
  q.pos = pos;
  q.req = n_tok > 1 ? (const int32_t*)pos : nullptr;   // (validation only: listed per request)
  q.max_pos = max_pos;
  hsa_status s;
  if ((s = check_attn_common(&q, Q, L->H, L->d, &L->ring_k, &L->ring_v, L->n_win, &L->kc, &L->vc,
                             L->m, L->scale, O)) != HSA_OK)
    return s;
  REQ(L->ring_k.capacity >= L->n_win + n_tok - 1 && L->ring_v.capacity >= L->n_win + n_tok - 1,
      "decode: rings must hold n_win + n_tok - 1 tokens");
  int64_t pages_needed = (max_pos + 1) / L->m;
  REQ((int64_t)L->kc.pages_per_req * kPage >= pages_needed &&
          (int64_t)L->vc.pages_per_req * kPage >= pages_needed,
      "decode: page table too short for the appended entries");
  if (L->kind == HSA_LAYER_CSA) {
    REQ(qI && kI_new && w && L->alpha_i, "decode: CSA needs qI, kI_new, w and alpha_i");
    if ((s = check_paged(&L->kic, "kic", kDI, false, false, true)) != HSA_OK) return s;
    SUP(L->kic.dtype != HSA_FP4_E2M1_MX || n_tok == 1,
        "decode: fp4 indexer keys take one token per request (no drafts)");
    // a draft's rejected tokens must not overwrite a kept token of the open
    // block (hsa_decode_rewind): the tail holds m + n_tok - 1 rows
    if ((s = check_tokens(&L->tail_i, "tail_i", kDI, L->m + n_tok - 1)) != HSA_OK) return s;
    REQ(L->kic.n_req >= B && L->tail_i.n_req >= B, "decode: kic holds fewer than B requests");
    REQ((int64_t)L->kic.pages_per_req * kPage >= pages_needed, "decode: kic table too short");
    SUP(L->H_I == kHI && L->d_I == kDI, "decode: H_I must be 4 and d_I 64");
    REQ(L->topk >= 1 && L->topk <= (1 << 20), "decode: topk out of range");
    SUP(nvis_host(max_pos, L->m, L->n_win) <= indexer_max_blocks(),
        "decode: rows longer than 2^21 visible blocks are not supported");
  }
  return HSA_OK;
}

hsa_status hsa_decode_step(const hsa_layer* L, int32_t B, const int64_t* pos, int64_t max_pos,
                           const void* Q, const void* k_new, const void* v_new, const void* qI,
                           const void* kI_new, const float* w, void* O, float* lse,
                           int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  hsa_status s;
  if ((s = check_decode(L, B, 1, pos, max_pos, Q, k_new, v_new, qI, kI_new, w, O)) != HSA_OK)
    return s;
  hsa_queries q{};
  q.n = B;
  q.pos = pos;
  q.max_pos = max_pos;
  const bool csa = L->kind == HSA_LAYER_CSA;
  size_t a_idx, a_sel, a_attn;
  decode_parts(L, B, max_pos, &a_idx, &a_sel, &a_attn);
  const size_t a_q = rope_q_bytes(L, (size_t)B);
  if ((s = check_ws(ws, ws_bytes, a_idx + a_sel + a_attn + a_q)) != HSA_OK) return s;
  char* base = (char*)ws;
  // RoPE: the upkeep writes the turned queries here, and the attention reads them
  void* q_rot = a_q ? base + a_idx + a_sel + a_attn : nullptr;
  const void* Qa = a_q ? q_rot : Q;
  hipError_t e;
  if (csa) {
    // the cache upkeep rides in one of the indexer's launches (which one
    // depends on the cache formats and the row length: launch_indexer); the
    // block completed at pos starts inside the window, so no query of this
    // step sees it and the scan never reads what the upkeep writes
    const UpdateArgs upd = make_update_args(*L, pos, max_pos, k_new, v_new, kI_new, Q, q_rot);
    int32_t* sel = idx_out ? idx_out : (int32_t*)(base + a_idx);
    e = launch_indexer(q, qI, w, L->kic, L->m, L->n_win, L->topk, sel, nullptr, base, a_idx,
                       stream, &upd);
    if (e != hipSuccess) return hip_status(e, "decode_step indexer");
    e = launch_attn(q, Qa, L->H, L->ring_k, L->ring_v, L->n_win, L->kc, L->vc, L->m, sel,
                    L->topk, L->scale, O, L->o_dtype, lse, base + a_idx + a_sel, a_attn, stream);
  } else if (a_q) {
    // RoPE: the attention needs the turned key and queries the upkeep writes
    e = launch_decode_update(*L, B, pos, max_pos, k_new, v_new, kI_new, stream, 1, nullptr,
                             nullptr, Q, q_rot);
    if (e != hipSuccess) return hip_status(e, "decode_step update");
    e = launch_attn(q, Qa, L->H, L->ring_k, L->ring_v, L->n_win, L->kc, L->vc, L->m, nullptr, 0,
                    L->scale, O, L->o_dtype, lse, base, a_attn, stream);
  } else {
    // the block completed at pos is not visible to the query at pos, so the
    // upkeep may follow the attention (in its merge launch): launch_attn
    // places it
    const UpdateArgs upd = make_update_args(*L, pos, max_pos, k_new, v_new, kI_new);
    e = launch_attn(q, Q, L->H, L->ring_k, L->ring_v, L->n_win, L->kc, L->vc, L->m, nullptr, 0,
                    L->scale, O, L->o_dtype, lse, base, a_attn, stream, &upd);
  }
  return hip_status(e, "decode_step attention");
}

// Draft queries of one request share the passes over its keys, up to four at
// a time: the largest divisor of n_tok not above 4.
static int draft_group(int n_tok) {
  return n_tok % 4 == 0 ? 4 : n_tok % 3 == 0 ? 3 : n_tok % 2 == 0 ? 2 : 1;
}

// Workspace of a draft: the queries' positions and requests, then the
// indexer's (in the grouped scan's shape), the selection's and the
// attention's parts for B * n_tok queries.
static void draft_parts(const hsa_layer* L, int32_t B, int32_t n_tok, int64_t max_pos,
                        size_t* p_q, size_t* p_idx, size_t* p_sel, size_t* p_attn) {
  const size_t n = (size_t)B * n_tok;
  hsa_queries q{};
  q.n = (int32_t)n;
  q.pos = (const int64_t*)1;   // list mode for sizing only
  q.req = (const int32_t*)1;
  q.max_pos = max_pos;
  *p_q = rnd256(sizeof(int64_t) * n) + rnd256(sizeof(int32_t) * n);
  *p_idx = *p_sel = 0;
  if (L->kind == HSA_LAYER_CSA) {
    *p_idx = rnd256(indexer_ws_bytes((int)n, nvis_host(max_pos, L->m, L->n_win), L->topk, false,
                                     draft_group(n_tok)));
    *p_sel = rnd256(sizeof(int32_t) * n * L->topk);
    *p_attn = rnd256(hsa_csa_attn_workspace_bytes(&q, L->H, L->n_win, L->topk));
  } else {
    *p_attn = rnd256(hsa_hca_attn_workspace_bytes(&q, L->H, L->n_win, L->m));
  }
}

size_t hsa_decode_draft_workspace_bytes(const hsa_layer* L, int32_t B, int32_t n_tok,
                                        int64_t max_pos) {
  if (!L || B < 1 || n_tok < 1 || max_pos < 0 || L->m < 1 || L->n_win < 1 || L->H < 16) return 0;
  if (L->kind == HSA_LAYER_CSA && L->topk < 1) return 0;
  size_t a, b, c, d;
  draft_parts(L, B, n_tok, max_pos, &a, &b, &c, &d);
  return a + b + c + d + rope_q_bytes(L, (size_t)B * n_tok);
}

hsa_status hsa_decode_draft(const hsa_layer* L, int32_t B, int32_t n_tok, const int64_t* pos,
                            int64_t max_pos, const void* Q, const void* k_new, const void* v_new,
                            const void* qI, const void* kI_new, const float* w, void* O,
                            float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  hsa_status s;
  if ((s = check_decode(L, B, n_tok, pos, max_pos, Q, k_new, v_new, qI, kI_new, w, O)) != HSA_OK)
    return s;
  size_t a_q, a_idx, a_sel, a_attn;
  draft_parts(L, B, n_tok, max_pos, &a_q, &a_idx, &a_sel, &a_attn);
  const size_t n = (size_t)B * n_tok;
  const size_t a_rq = rope_q_bytes(L, n);
  if ((s = check_ws(ws, ws_bytes, a_q + a_idx + a_sel + a_attn + a_rq)) != HSA_OK) return s;
  char* base = (char*)ws;
  int64_t* q_pos = (int64_t*)base;
  int32_t* q_req = (int32_t*)(base + rnd256(sizeof(int64_t) * n));
  void* q_rot = a_rq ? base + a_q + a_idx + a_sel + a_attn : nullptr;
  const void* Qa = a_rq ? q_rot : Q;
  // 1-2: every draft token appended in order (rings, tail, completed blocks);
  // the queries' positions and requests (and, with RoPE, the turned queries)
  // land in the workspace
  hipError_t e = launch_decode_update(*L, B, pos, max_pos, k_new, v_new, kI_new, stream, n_tok,
                                      q_pos, q_req, Q, q_rot);
  if (e != hipSuccess) return hip_status(e, "decode_draft update");
  // 3: query i of request b at position pos[b] + i sees exactly what a
  // single-token step at that position would (a block completed later in the
  // draft is not visible to it; its window rows survive in the ring)
  hsa_queries q{};
  q.n = (int32_t)n;
  q.pos = q_pos;
  q.req = q_req;
  q.max_pos = max_pos;
  if (L->kind == HSA_LAYER_CSA) {
    int32_t* sel = idx_out ? idx_out : (int32_t*)(base + a_q + a_idx);
    e = launch_indexer(q, qI, w, L->kic, L->m, L->n_win, L->topk, sel, nullptr, base + a_q,
                       a_idx, stream, nullptr, draft_group(n_tok));
    if (e != hipSuccess) return hip_status(e, "decode_draft indexer");
    e = launch_attn(q, Qa, L->H, L->ring_k, L->ring_v, L->n_win, L->kc, L->vc, L->m, sel,
                    L->topk, L->scale, O, L->o_dtype, lse, base + a_q + a_idx + a_sel, a_attn,
                    stream);
  } else {
    e = launch_attn(q, Qa, L->H, L->ring_k, L->ring_v, L->n_win, L->kc, L->vc, L->m, nullptr, 0,
                    L->scale, O, L->o_dtype, lse, base + a_q, a_attn, stream);
  }
  return hip_status(e, "decode_draft attention");
}

hsa_status hsa_decode_rewind(const hsa_layer* L, int32_t B, const int64_t* keep,
                             hipStream_t stream) {
  REQ(L, "decode_rewind: null layer");
  REQ(L->kind == HSA_LAYER_CSA || L->kind == HSA_LAYER_HCA, "decode_rewind: unknown layer kind");
  REQ(B >= 1 && keep, "decode_rewind: null keep or B < 1");
  REQ(L->m >= 1, "decode_rewind: bad m");
  hsa_status s;
  if ((s = check_paged(&L->kc, "kc", kD, true, true)) != HSA_OK) return s;
  if ((s = check_paged(&L->vc, "vc", kD, true)) != HSA_OK) return s;
  if ((s = check_append_caches(L, "decode_rewind")) != HSA_OK) return s;
  REQ(L->kc.n_req >= B && L->vc.n_req >= B, "decode_rewind: caches hold fewer than B requests");
  if (L->kind == HSA_LAYER_CSA) {
    if ((s = check_paged(&L->kic, "kic", kDI, false, false, true)) != HSA_OK) return s;
    REQ(L->kic.n_req >= B, "decode_rewind: kic holds fewer than B requests");
  }
  return hip_status(launch_decode_rewind(*L, B, keep, stream), "decode_rewind");
}

hsa_status hsa_decode_step_noalloc(const hsa_layer* L, int32_t B, const int64_t* pos,
                                   int64_t max_pos, const void* Q, const void* k_new,
                                   const void* v_new, const void* qI, const void* kI_new,
                                   const float* w, void* O, float* lse, int32_t* idx_out,
                                   hipStream_t stream) {
  const size_t need = hsa_decode_step_workspace_bytes(L, B, max_pos);
  if (need > HSA_NOALLOC_SCRATCH_BYTES)
    return fail(HSA_ERR_WORKSPACE,
                "decode_step_noalloc: this step needs " + std::to_string(need) +
                    " bytes of workspace, more than the library's " +
                    std::to_string((size_t)HSA_NOALLOC_SCRATCH_BYTES) + "-byte scratch");
  void* ws = scratch_ptr();
  if (!ws) return fail(HSA_ERR_HIP, "decode_step_noalloc: no scratch address on this device");
  // the decode workspace needs no clearing: every call writes what it reads
  return hsa_decode_step(L, B, pos, max_pos, Q, k_new, v_new, qI, kI_new, w, O, lse, idx_out, ws,
                         HSA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
