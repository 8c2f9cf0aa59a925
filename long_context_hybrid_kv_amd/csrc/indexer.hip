// Lightning indexer and per-query top-k selection (CSA).
//
// Score of block b for query t: I = sum_h w[t][h] * max(0, qI[t][h] . KI_c[b]),
// h < 4, d_I = 64, fp32 accumulation of bf16 products.  The dot products run on
// MFMA 16x16x32 bf16 tiles: the A operand holds query-heads as rows (4 query
// tokens x 4 heads in prefill; one query's 4 heads and 12 zero rows in decode),
// the B operand holds 16 compressed indexer keys, so each lane of the result
// owns the 4 heads of one (query, block) pair and the head sum stays in-lane.
// bf16 keys load as whole 128-byte rows (8 keys per load instruction) into a
// per-wave swizzled LDS tile and are read back in the MFMA B layout (fp8 keys
// load as pieces and widen in registers); prefill also stages the A operand
// (queries) in LDS.  Over fp4 keys
// (OCP MX FP4) the indexer computes in FP4: each query head is quantized to
// MX FP4 by the keys' own rule, and the 16x16x128 MX-scaled MFMA takes both
// operands as e2m1 codes with their e8m0 block scales (every product exact,
// fp32 accumulation); the upper half of its 128-deep operands meets zero
// query codes.
//
// Selection is exact, with no synchronisation between workgroups inside a
// kernel (on this multi-XCD chip a device-scope fence per workgroup costs more
// than the whole score stream).  Every path begins with
//   scan     fp32 scores into the workspace, and a histogram of the top 12 bits
//            of the order-preserving score key per chunk in LDS.
// Decode rows of more than kFusedMaxBlocksDecode blocks then take the
// candidate path, two kernels in all:
//   scan     also hands over, per workgroup, the nonzero bins at or above the
//            bin of its c-th largest score (c ~ 3k / workgroups) and the keys
//            in them (at most kCandCap);
//   cand     one workgroup per query merges those bin lists into the row's
//            histogram above the cut, finds the bin holding the k-th largest
//            score, and settles the selection from the candidate union alone:
//            bins above it are taken whole, the threshold bin is refined with
//            radix passes over the rest of the key (ties -> lower block).  If
//            the union cannot prove the answer (a workgroup's cut lies at or
//            above the threshold bin, or a list overflowed) the workgroup
//            selects over the whole row instead.
// Prefill, and rows too long for the bitmap in LDS, take three kernels:
//   select   every chunk finds, from the per-query histogram, the bin holding
//            the k-th largest score, marks its blocks above that bin in a
//            per-query bitmap and appends the blocks inside it to a candidate
//            list;
//   finalize one workgroup per query refines the candidates with 8-bit radix
//            passes over the rest of the score key and then over the inverted
//            block index (ties -> lower block), and emits the bitmap in
//            ascending block order.
// The workspace needs no clearing between calls: histogram and candidate lists
// are rewritten whole by the kernels that produce them, and the per-query
// counters are reset by the kernel that owns them before their first use.
#include <type_traits>

#include "update.h"

namespace hsa {

constexpr int kCH = 512;           // blocks per scan chunk
// chunks per scan workgroup (one histogram list each): long rows group 4 chunks
// so that the threshold pass merges 4x fewer lists
constexpr int kLongRowChunks = 256;
static int scan_cpw(int64_t R) { return R / kCH >= kLongRowChunks ? 4 : 1; }
constexpr int kSelCH = 2048;       // blocks per select workgroup (multiple of kCH)
constexpr int kMaxSelChunks = 1024;  // select chunks whose offsets fit in LDS
constexpr int kGemmMaxPages = 1024;  // pages of a prefill score workgroup resolved in LDS
constexpr int kBins = 4096;        // first-level histogram (12 key bits)
constexpr int kBmLdsMaxWords = 16384;  // refine pass: bitmaps up to this size go to LDS
constexpr int kSpanQC = 2048;      // prefill: queries per workspace pass
// per-query state: [2] threshold bin, [3] blocks above it, [5] visible blocks,
// [6] blocks in the threshold bin; the candidate path records instead in [6]
// which selection served the query (0 the union; the whole row: 1 a list
// overflowed, 2 no threshold bin, 3 a workgroup's cut at or above it, 4 the
// threshold bin holds more than kThrCandMax) and in [7] the union size << 16 |
// threshold-bin size
constexpr int kStateInts = 8;
constexpr int kHistSpan = 8192;    // prefill: scores per histogram workgroup
// decode candidate selection (long rows): each scan workgroup hands over the
// scores in the histogram bins down to the one holding its c-th largest, at
// most kCandCap of them; one workgroup per query selects from their union
constexpr int kCandCap = 256;      // candidates a scan workgroup may write
constexpr int kTopBins = 16;       // nonzero bins >= its cut bin a scan workgroup may list
constexpr int kCandBmMaxWords = 16384;   // bitmap words of the emission in LDS
constexpr int kThrCandMax = 4096;  // candidates of the threshold bin the selection refines in LDS
constexpr int kCandMaxLists = 256;  // scan workgroups (lists) of a query the selection merges

struct IdxWs {
  float* scores;        // [nq][R]
  uint32_t* hl;         // [nq][n_lists][list_cap] histogram lists: bin << 16 | count
  int32_t* hl_n;        // [nq][n_lists] entries of each list
  int32_t* state;       // [nq][kStateInts]
  uint32_t* bitmap;     // [nq][R/32]
  uint64_t* cand;       // [nq][R]  (score key << 32 | ~block)
  uint64_t* cand2;      // [nq][R]
  int32_t* ccount;      // [nq][R/kSelCH]  candidates per select chunk (long rows)
  uint64_t* wcand;      // decode, listed queries: [nq][n_lists][kCandCap] candidate keys
  int32_t* wcnt;        // [nq][n_lists] candidates each scan workgroup found (> kCandCap: overflow)
  int32_t* wbin;        // [nq][n_lists] its cut bin: every score left out lies in a lower bin (-1: none)
  uint32_t* wtop;       // [nq][n_lists][kTopBins] its nonzero bins >= the cut bin: bin << 16 | count
  int32_t* wntop;       // [nq][n_lists] entries of that list (> kTopBins: overflow)
  int64_t R;
  int n_lists;          // one list per scan chunk (decode) or histogram slice (prefill)
  int list_cap;         // nonzero bins a list can hold
  int list_span;        // scores a list covers
};

static int64_t row_cap(int64_t max_nvis) {
  int64_t R = ((max_nvis + kSelCH - 1) / kSelCH) * kSelCH;
  return R < kSelCH ? kSelCH : R;
}

static void list_shape(int64_t R, bool span, int* n_lists, int* cap, int* span_len,
                       bool grouped = false) {
  *span_len = span ? kHistSpan : (grouped ? 1 : scan_cpw(R)) * kCH;
  *n_lists = (int)((R + *span_len - 1) / *span_len);
  *cap = *span_len < kBins ? *span_len : kBins;   // at most min(bins, scores) entries
}

// The workspace layout, walked once for sizing (base == nullptr) and once for
// carving, so the two can never disagree.  grouped: the draft scan's shape
// (one histogram list per 512-block chunk at every row length).
static size_t layout(char* base, int nq, int64_t R, bool span, bool grouped, IdxWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = base ? base + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return r;
  };
  list_shape(R, span, &w->n_lists, &w->list_cap, &w->list_span, grouped);
  w->state = (int32_t*)take(sizeof(int32_t) * kStateInts * nq);
  w->hl_n = (int32_t*)take(sizeof(int32_t) * w->n_lists * nq);
  w->hl = (uint32_t*)take(sizeof(uint32_t) * w->list_cap * w->n_lists * nq);
  w->scores = (float*)take(sizeof(float) * R * nq);
  w->bitmap = (uint32_t*)take(sizeof(uint32_t) * (R / 32) * nq);
  w->cand = (uint64_t*)take(sizeof(uint64_t) * R * nq);
  w->cand2 = (uint64_t*)take(sizeof(uint64_t) * R * nq);
  w->ccount = (int32_t*)take(sizeof(int32_t) * (R / kSelCH) * nq);
  const bool cand = !span && !grouped;
  w->wcand = cand ? (uint64_t*)take(sizeof(uint64_t) * kCandCap * w->n_lists * nq) : nullptr;
  w->wcnt = cand ? (int32_t*)take(sizeof(int32_t) * w->n_lists * nq) : nullptr;
  w->wbin = cand ? (int32_t*)take(sizeof(int32_t) * w->n_lists * nq) : nullptr;
  w->wtop = cand ? (uint32_t*)take(sizeof(uint32_t) * kTopBins * w->n_lists * nq) : nullptr;
  w->wntop = cand ? (int32_t*)take(sizeof(int32_t) * w->n_lists * nq) : nullptr;
  w->R = R;
  return off;
}

static size_t carve_bytes(int nq, int64_t R, bool span, bool grouped) {
  IdxWs w;
  return layout(nullptr, nq, R, span, grouped, &w);
}

static int64_t host_nvis(int64_t t, int m, int n_win) {
  int64_t s = t - n_win + 1 < 0 ? 0 : t - n_win + 1;
  int64_t a = (s + m - 1) / m, b = (t + 1) / m;
  return a < b ? a : b;
}

size_t indexer_ws_bytes(int n_q, int64_t max_nvis, int k, bool span, int group) {
  (void)k;
  int nq = span ? (n_q < kSpanQC ? n_q : kSpanQC) : n_q;
  return carve_bytes(nq, row_cap(max_nvis), span, !span && group > 1);
}

// decode rows up to 2^21 visible blocks (an 8M-token context at m = 4)
int64_t indexer_max_blocks() { return int64_t(1) << 21; }

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// candidate keys rewritten by this workgroup between passes: device-coherent
// loads (LDS or L2), never a stale vector-L1 line
__device__ __forceinline__ uint64_t ld_cand(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Index scores in the workspace: fp32, or (S16) rounded once to bf16, round
// to nearest even, where the selection runs on bf16 scores (the wiki's bf16
// selector).  Row q holds R scores.  Scores are rounded before they are
// histogrammed, so every pass of the selection sees the same values.
template <bool S16>
__device__ __forceinline__ float score_round(float s) {
  if constexpr (S16) return (float)(__bf16)s;
  else return s;
}
template <bool S16>
__device__ __forceinline__ void* score_row(const IdxWs& ws, int64_t q) {
  return (char*)ws.scores + q * ws.R * (S16 ? 2 : 4);
}
template <bool S16>
__device__ __forceinline__ float score_load(const void* row, int64_t i) {
  if constexpr (S16) return __uint_as_float((uint32_t)((const u16*)row)[i] << 16);
  else return ((const float*)row)[i];
}
template <bool S16>   // s: a value score_round returned
__device__ __forceinline__ void score_store(void* row, int64_t i, float s) {
  if constexpr (S16) ((u16*)row)[i] = (u16)(__float_as_uint(s) >> 16);
  else ((float*)row)[i] = s;
}
// Score i of a row if i < lim, for a caller that ignores the value otherwise:
// fp32 rows read 0 past lim; bf16 rows clamp the index to the row's capacity
// R instead, so their 16-bit loads need no branch (a branch around each one
// made the compiler wait for every load before the next).
template <bool S16>
__device__ __forceinline__ float score_get(const void* row, int64_t i, int64_t lim, int64_t R) {
  if constexpr (S16) return score_load<true>(row, i < R ? i : R - 1);
  else return i < lim ? ((const float*)row)[i] : 0.f;
}

// exclusive prefix sum over a 256-thread block; returns the block total in *total
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t s = sh[i];
    if (i < wv) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

__device__ __forceinline__ int64_t clamp_nvis(int64_t nv, const int32_t* n_entries, int r,
                                              int* fault, bool report) {
  int64_t ne = n_entries[r];
  if (nv > ne) {
    if (report) atomicOr(fault, HSA_FAULT_ENTRIES);
    nv = ne < 0 ? 0 : ne;
  }
  return nv;
}

// bitwise AND and OR of 64-bit values over an NT-thread block (every thread
// gets both totals; sh64 holds 2 * NT / 64 words)
template <int NT>
__device__ __forceinline__ void block_and_or(uint64_t* a, uint64_t* o, uint64_t* sh64) {
  uint32_t alo = (uint32_t)*a, ahi = (uint32_t)(*a >> 32);
  uint32_t olo = (uint32_t)*o, ohi = (uint32_t)(*o >> 32);
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    alo &= __shfl_xor(alo, d);
    ahi &= __shfl_xor(ahi, d);
    olo |= __shfl_xor(olo, d);
    ohi |= __shfl_xor(ohi, d);
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    sh64[wv] = ((uint64_t)ahi << 32) | alo;
    sh64[NT / 64 + wv] = ((uint64_t)ohi << 32) | olo;
  }
  __syncthreads();
  uint64_t x = ~0ull, y = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    x &= sh64[i];
    y |= sh64[NT / 64 + i];
  }
  __syncthreads();   // sh64 is reused
  *a = x;
  *o = y;
}

// exclusive prefix sum over an NT-thread block (NT a multiple of 64)
template <int NT>
__device__ __forceinline__ uint32_t block_scan_nt(uint32_t v, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    uint32_t s = sh[i];
    if (i < wv) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// Write a 4096-bin LDS histogram (a workgroup of NTH threads) as a list of its
// nonzero bins, bin << 16 | count, into list `li` of query row `qrow`.  Lists
// are rewritten whole by every call, so the workspace needs no clearing
// between calls.
template <int NTH = 256>
__device__ __forceinline__ void write_hist_list(const uint32_t* lhist, const IdxWs& ws, int qrow,
                                                int li) {
  __shared__ uint32_t sh[NTH / 64];
  __syncthreads();
  constexpr int BPT = kBins / NTH;
  uint32_t v[BPT];
  uint32_t nz = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {   // thread t owns bins t, t + NTH, ... (no bank conflicts)
    v[j] = lhist[threadIdx.x + NTH * j];
    nz += v[j] != 0;
  }
  uint32_t tot;
  uint32_t off = block_scan_nt<NTH>(nz, &tot, sh);
  uint32_t* dst = ws.hl + ((int64_t)qrow * ws.n_lists + li) * ws.list_cap;
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if (v[j]) dst[off++] = ((uint32_t)(threadIdx.x + NTH * j) << 16) | v[j];
  if (threadIdx.x == 0) ws.hl_n[(int64_t)qrow * ws.n_lists + li] = (int32_t)tot;
}

// Candidates of one scan workgroup (decode, long rows): the cut bin b_c is the
// highest bin of the workgroup's 4096-bin histogram whose count from the top
// reaches c_local; every score in a bin >= b_c is written as a key
// (score key << 32 | ~block), at most kCandCap of them, and every score left
// out lies in a bin below b_c.  wcnt records how many there were (more than
// kCandCap: the selection falls back to the full row), wbin the cut bin (-1
// when nothing was left out), wtop the nonzero bins >= b_c with their counts
// (in no particular order; the selection merges them as a set) and wntop how
// many there were.  n_sc scores in lsc (LCAP slots) belong to blocks s0 ...
template <int NTH, int LCAP>
__device__ __forceinline__ void write_candidates(const uint32_t* lhist, const float* lsc, int n_sc,
                                                 int64_t s0, const IdxWs& ws, int qrow, int wg,
                                                 int c_local) {
  __shared__ uint32_t sh[NTH / 64];
  __shared__ int s_bc;
  __shared__ uint32_t s_n;
  constexpr int BPT = kBins / NTH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t li = (int64_t)qrow * ws.n_lists + wg;
  const int lo = kBins - BPT * (tid + 1);        // thread 0 owns the highest bins
  uint32_t v[BPT], sm = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    v[j] = lhist[lo + j];
    sm += v[j];
  }
  if (tid == 0) { s_bc = 0; s_n = 0; }
  uint32_t tot;
  const uint32_t pre = block_scan_nt<NTH>(sm, &tot, sh);
  if (pre < (uint32_t)c_local && pre + sm >= (uint32_t)c_local) {
    uint32_t cum = pre;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (cum < (uint32_t)c_local && cum + v[j] >= (uint32_t)c_local) s_bc = lo + j;
      cum += v[j];
    }
  }
  __syncthreads();
  const int bc = s_bc;                           // 0 when the workgroup holds fewer scores
  // Two lists, each compacted with one wave scan and one atomic per wave on a
  // packed counter (bins << 16 | candidates, both below 2^16): the thread's
  // nonzero bins >= bc (held in v[]), and its candidates -- PER of the LCAP
  // slots of lsc, read whether or not they hold a score so that no read waits
  // behind a branch
  constexpr int PER = LCAP / NTH;
  static_assert(PER >= 1 && PER * NTH == LCAP && LCAP < 65536 && kBins < 65536, "packed counts");
  uint32_t key[PER], cnt = 0, nb = 0;
  bool c[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) key[j] = order_key(lsc[tid + NTH * j]);
#pragma unroll
  for (int j = 0; j < BPT; ++j) nb += (lo + j >= bc && v[j] != 0);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = tid + NTH * j < n_sc && (int)(key[j] >> 20) >= bc;
    cnt += c[j];
  }
  const uint32_t mine = (nb << 16) | cnt;
  const uint32_t inc = wave_incl_sum(mine);
  const uint32_t wtot = lane_value(inc, 63);
  uint32_t wb = 0;
  if (wtot != 0) {   // uniform in the wave
    if (lane == 0) wb = atomicAdd(&s_n, wtot);
    wb = lane_value(wb, 0);
  }
  const uint32_t base = wb + inc - mine;
  uint32_t pos = base & 0xFFFFu, ob = base >> 16;
  uint64_t* dst = ws.wcand + li * kCandCap;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (c[j]) {
      if (pos < (uint32_t)kCandCap)
        dst[pos] = ((uint64_t)key[j] << 32) | (uint64_t)(~(uint32_t)(s0 + tid + NTH * j));
      ++pos;
    }
  if (nb != 0 && ob < (uint32_t)kTopBins) {
    uint32_t* lst = ws.wtop + li * kTopBins;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j)
      if (lo + j >= bc && v[j] != 0) {
        if (ob < (uint32_t)kTopBins) lst[ob] = ((uint32_t)(lo + j) << 16) | v[j];
        ++ob;
      }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t n_c = s_n & 0xFFFFu;
    ws.wcnt[li] = (int32_t)n_c;
    ws.wntop[li] = (int32_t)(s_n >> 16);
    // anything below the cut bin left out?  (bins below bc hold tot - n_c scores)
    ws.wbin[li] = n_c < (uint32_t)n_sc ? bc : -1;
  }
}

// ---------------------------------------------------------------- decode: score scan

// F8K: fp8 keys with a page scale; F4K: fp4 keys (MX blocks); neither: bf16
template <int CPW, int NWV, bool F8K, bool F4K, bool S16>
__global__ __launch_bounds__(NWV * 64) void idx_scan_kernel(Queries Q, const u16* __restrict__ qI,
                                                       const float* __restrict__ w, Paged kic,
                                                       int m, int n_win, int k, IdxWs ws,
                                                       int n_groups, UpdateArgs upd, int cand_k,
                                                       int* fault) {
  const int qrow = blockIdx.y;
  if ((int)blockIdx.x >= n_groups) {   // the extra column: cache upkeep of request qrow
    decode_update_body<false>(upd, qrow, fault);   // bf16 caches, no RoPE (the host's rule)
    return;
  }
  const int c_first = blockIdx.x * CPW;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, row = lane & 15, g = lane >> 4;
  const int r8 = lane >> 3, p8 = lane & 7;   // bf16 loads: key r8 of 8, 16-byte piece p8
  // A workgroup of NWV waves scores CPW consecutive chunks of kCH blocks; in
  // each chunk a wave streams BPW consecutive blocks = PPW whole pages.  The
  // page ids depend only on the request, so they are loaded alongside the
  // query's position and entry count instead of after them: the key loads wait
  // for one round trip.
  constexpr int BPW = kCH / NWV, PPW = BPW / kPage;
  static_assert(PPW >= 1, "a wave streams whole pages");
  const int r = Q.req_of(qrow, fault);
  int pid[CPW][PPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int lp = (int)((((int64_t)(c_first + c)) * kCH + wv * BPW) >> 6);
#pragma unroll
    for (int j = 0; j < PPW; ++j)
      pid[c][j] = lp + j < kic.pages_per_req
                      ? kic.page_table[(int64_t)r * kic.pages_per_req + lp + j]
                      : -1;
  }
  // the entry count and the position, issued behind the page ids and moved to
  // scalar registers only once both are in flight: one wait for all of them
  const int z = opaque_zero();
  const int32_t ne_v = kic.n_entries[r + z];
  const int64_t p_v = Q.pos ? Q.pos[qrow + z] : 0;
  const int64_t ne = (int32_t)__builtin_amdgcn_readfirstlane(ne_v);
  int64_t t = Q.span_pos0 + qrow;
  if (Q.pos) {
    t = readfirstlane64(p_v);
    if (t > Q.max_pos || t < 0) {
      atomicOr(fault, HSA_FAULT_POS);
      t = t < 0 ? 0 : Q.max_pos;
    }
  }
  int64_t nv = n_visible(t, m, n_win);
  if (nv > ne) {
    if (c_first == 0 && threadIdx.x == 0) atomicOr(fault, HSA_FAULT_ENTRIES);
    nv = ne < 0 ? 0 : ne;
  }
  const int n_active = nv > 0 ? (int)((nv + kCH - 1) / kCH) : 1;
  if (c_first >= n_active) return;
  if (c_first == 0 && threadIdx.x == 0) ws.state[(int64_t)qrow * kStateInts + 5] = (int32_t)nv;

  constexpr int NT = BPW / 16;   // 16-block tiles per wave and chunk
  // key pieces of a lane, 16 bytes each: bf16, 8 channels (two pieces per
  // tile); fp8 codes, 16 channels (one piece per tile), widened to bf16 when
  // scored, the page scale applied to the head sum
  typedef typename std::conditional<F8K || F4K, u32x4, bf16x8>::type KeyT;
  float ksc[CPW][PPW];   // fp8: scale of the wave's pages of each chunk
  // branch-free loads (tile u lies in the wave's page u / 4)
  auto load = [&](int c, KeyT* x0, KeyT* x1) {
    const int64_t cb = (int64_t)(c_first + c) * kCH;
    const int64_t b_end = nv < cb + kCH ? nv : cb + kCH;
    const int64_t w0b = cb + (int64_t)wv * BPW;
    if constexpr (F8K) {
#pragma unroll
      for (int j = 0; j < PPW; ++j)
        ksc[c][j] = (unsigned)pid[c][j] < (unsigned)kic.n_pages ? kic.scale[pid[c][j]] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int pg = pid[c][u >> 2];
      const bool okp = (unsigned)pg < (unsigned)kic.n_pages;
      if constexpr (F8K) {
        // 64-byte keys: one load instruction reads 16 whole keys, lane (row, g)
        // channels 16g .. 16g+15 of key `row` (the query's channels are
        // permuted to match).  Keys past the row's end are read but never
        // scored; a bad page reads page 0.
        x0[u] = __builtin_nontemporal_load(
            (const KeyT*)(kic.data + ((int64_t)(okp ? pg : 0) * kPage + 16 * (u & 3) + row) * kDI) + g);
      } else if constexpr (F4K) {
        // 32-byte keys, the MFMA's B operand: lane (row, g) reads MX block g & 1
        // of key `row` (16 bytes, 32 channels) and its scale byte (x1[u].x);
        // lanes g >= 2 fill the 128-deep operand's upper half, which meets
        // zero query codes
        const int64_t er = (int64_t)(okp ? pg : 0) * kPage + 16 * (u & 3) + row;
        x0[u] = __builtin_nontemporal_load((const u32x4*)(kic.data + er * (kDI / 2)) + (g & 1));
        x1[u].x = ((const uint8_t*)kic.scale)[er * (kDI / 32) + (g & 1)];
      } else {
        // whole rows: each load instruction reads 8 consecutive 128-byte keys,
        // lane (r8, p8) piece p8 of key r8 (score() moves them to the MFMA
        // layout).  Tiles are page-aligned, so both loads stay in the page;
        // keys past the row's end are read but never scored, and a bad page
        // reads page 0.
        const KeyT* kr = (const KeyT*)(kic.data + ((int64_t)(okp ? pg : 0) * kPage +
                                                   16 * (u & 3) + r8) * (kDI * 2)) + p8;
        x0[u] = __builtin_nontemporal_load(kr);
        x1[u] = __builtin_nontemporal_load(kr + 8 * (kDI * 2 / 16));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < PPW; ++j)
        if (w0b + 64 * j < b_end && (unsigned)pid[c][j] >= (unsigned)kic.n_pages)
          atomicOr(fault, HSA_FAULT_PAGE);
    }
  };
  // query head `row` in the channel order of the keys: bf16, channels 8g..8g+7
  // then 32+8g..; fp8 and fp4, 16g..16g+7 then 16g+8..16g+15.  Requested
  // before the keys: loads complete in order, and the first chunk's scoring
  // waits for these, not for the keys of the chunks behind it.
  bf16x8 a0 = {}, a1 = {};
  if (!F4K && row < kHI) {   // (fp4: the query is quantized into LDS below)
    const bf16x8* qa = (const bf16x8*)(qI + ((int64_t)qrow * kHI + row) * kDI);
    a0 = qa[F8K ? 2 * g : g];
    a1 = qa[F8K ? 2 * g + 1 : 4 + g];
  }
  const float w0 = w[qrow * kHI + 0], w1 = w[qrow * kHI + 1], w2 = w[qrow * kHI + 2],
              w3 = w[qrow * kHI + 3];
  KeyT xa0[NT], xa1[NT], xb0[NT], xb1[NT];
  load(0, xa0, xa1);
  if (CPW > 1) load(1, xb0, xb1);
  // the LDS histogram is cleared while the keys are in flight
  __shared__ uint32_t lhist[kBins];
  __shared__ float lsc[CPW * kCH];
  __shared__ bf16x8 ltile[F8K ? 1 : NWV][F8K ? 1 : 128];   // bf16: one 16-key tile per wave
  for (int i = threadIdx.x; i < kBins; i += NWV * 64) lhist[i] = 0;
  // fp4: the query heads in MX FP4 (the indexer computes in FP4), quantized
  // once per workgroup into LDS, then the MFMA's A operand: lane (row, g < 2)
  // holds block g of head `row`; the other lanes zero codes with scale 1
  __shared__ __align__(16) uint32_t qcodes[F4K ? kHI : 1][8];
  __shared__ uint8_t qsb[F4K ? kHI : 1][2];
  if constexpr (F4K) mx_fp4_rows(qI + (int64_t)qrow * kHI * kDI, kHI, kHI, qcodes, qsb);
  __syncthreads();
  u32x4 qf = {0u, 0u, 0u, 0u};
  uint32_t qs = 127u;
  if constexpr (F4K)
    if (row < kHI && g < 2) {
      qf = *(const u32x4*)&qcodes[row][4 * g];
      qs = qsb[row][g];
    }

  auto score = [&](int c, const KeyT* x0, const KeyT* x1) {
    const int64_t cb = (int64_t)(c_first + c) * kCH;
    const int64_t b_end = nv < cb + kCH ? nv : cb + kCH;
    const int64_t w0b = cb + (int64_t)wv * BPW;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      bf16x8 k0, k1;
      if constexpr (F8K) {
        k0 = e4m3x8_to_bf16x8(x0[u].xy);   // channels 16g .. 16g+7
        k1 = e4m3x8_to_bf16x8(x0[u].zw);   // channels 16g+8 .. 16g+15
      } else if constexpr (F4K) {
        // (scored by the MX FP4 MFMA below)
      } else {
        // the wave's 16 keys through its LDS tile: piece p of key r is stored
        // at slot p ^ (r & 7), so the row-wise writes and the MFMA-layout
        // reads both spread over all banks.  LDS executes a wave's accesses
        // in order; the asm statements keep the compiler from moving them
        // past each other (lanes read what other lanes wrote).
        asm volatile("" ::: "memory");
        ltile[wv][r8 * 8 + (p8 ^ r8)] = x0[u];
        ltile[wv][(8 + r8) * 8 + (p8 ^ r8)] = x1[u];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        k0 = ltile[wv][row * 8 + (g ^ (row & 7))];
        k1 = ltile[wv][row * 8 + ((4 + g) ^ (row & 7))];
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F4K) {
        acc = mfma_mx_fp4(qf, qs, x0[u], x1[u].x, acc);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, k0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, k1, acc, 0, 0, 0);
      }
      const int64_t b = w0b + 16 * u + row;
      if (g == 0 && b < b_end) {
        float sc = w0 * fmaxf(acc[0], 0.f) + w1 * fmaxf(acc[1], 0.f) +
                   w2 * fmaxf(acc[2], 0.f) + w3 * fmaxf(acc[3], 0.f);
        if constexpr (F8K) sc *= ksc[c][u >> 2];   // ReLU commutes with a scale > 0
        sc = score_round<S16>(sc);
        lsc[b - (int64_t)c_first * kCH] = sc;
        atomicAdd(&lhist[order_key(sc) >> 20], 1u);
      }
    }
  };
  // two register buffers: the next chunk's keys load while this one is scored
#pragma unroll
  for (int c = 0; c < CPW; c += 2) {
    score(c, xa0, xa1);
    if (c + 2 < CPW) load(c + 2, xa0, xa1);
    if (c + 1 < CPW) {
      score(c + 1, xb0, xb1);
      if (c + 3 < CPW) load(c + 3, xb0, xb1);
    }
  }
  __syncthreads();
  // the scores leave in one coalesced run
  void* srow = score_row<S16>(ws, qrow);
  const int64_t s0 = (int64_t)c_first * kCH;
  const int64_t s_end = nv < s0 + CPW * kCH ? nv : s0 + CPW * kCH;
  for (int i = threadIdx.x; i < CPW * kCH; i += NWV * 64)
    if (s0 + i < s_end) score_store<S16>(srow, s0 + i, lsc[i]);
  if (cand_k > 0) {
    // candidates per workgroup: three times the query's top-k spread over its
    // workgroups (so one workgroup rarely holds more of the top-k than it hands
    // over), at least 16, at most half the candidate space
    const int n_act = (n_active + CPW - 1) / CPW;
    int c_local = (3 * cand_k + n_act - 1) / n_act;
    c_local = c_local < 16 ? 16 : (c_local > kCandCap / 2 ? kCandCap / 2 : c_local);
    write_candidates<NWV * 64, CPW * kCH>(lhist, lsc, (int)(s_end - s0), s0, ws, qrow, blockIdx.x, c_local);
  } else
    write_hist_list<NWV * 64>(lhist, ws, qrow, blockIdx.x);
}

// Write a histogram of 16-bit counts packed two bins per word (bin b in half
// b & 1 of word b >> 1) as the list of its nonzero bins, like write_hist_list.
__device__ __forceinline__ void write_hist_list16(const uint32_t* lh2, const IdxWs& ws, int qrow,
                                                  int li) {
  __shared__ uint32_t sh[4];
  __syncthreads();
  constexpr int BPT = kBins / 256;
  uint32_t v[BPT];
  uint32_t nz = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = threadIdx.x + 256 * j;
    v[j] = (lh2[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu;
    nz += v[j] != 0;
  }
  uint32_t tot;
  uint32_t off = block_scan_nt<256>(nz, &tot, sh);
  uint32_t* dst = ws.hl + ((int64_t)qrow * ws.n_lists + li) * ws.list_cap;
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if (v[j]) dst[off++] = ((uint32_t)(threadIdx.x + 256 * j) << 16) | v[j];
  if (threadIdx.x == 0) ws.hl_n[(int64_t)qrow * ws.n_lists + li] = (int32_t)tot;
}

// ---------------------------------------------------------------- decode drafts: grouped scan

// Listed queries in groups of G (2..4) consecutive queries of one request, as
// a decode draft lays them out.  The MFMA A tile has 16 rows and one query
// fills four (its indexer heads), so the group's queries take rows 4i..4i+3
// and one pass over the request's keys scores all of them: lane group i
// (lanes 16i..16i+15) receives query i's four head products of its blocks.
// Per query, as idx_scan_kernel: the fp32 scores of its visible blocks and the
// nonzero bins of a 4096-bin histogram as list blockIdx.x (one 512-block chunk
// per workgroup; counts <= 512, so 16-bit bins, two per word, keep the G
// histograms small).
template <int G, bool F8K>
__global__ __launch_bounds__(256) void idx_scan_group_kernel(Queries Q, const u16* __restrict__ qI,
                                                             const float* __restrict__ w,
                                                             Paged kic, int m, int n_win,
                                                             IdxWs ws, int* fault) {
  const int q0 = blockIdx.y * G;
  const int c_first = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, row = lane & 15, g = lane >> 4;
  const int r = Q.req_of(q0, fault);
  int pid[2];
  {
    const int lp = (int)((((int64_t)c_first) * kCH + wv * (kCH / 4)) >> 6);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pid[j] = lp + j < kic.pages_per_req ? kic.page_table[(int64_t)r * kic.pages_per_req + lp + j]
                                          : -1;
  }
  int64_t nvq[G], nv_max = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    int rq;
    int64_t t;
    Q.get(q0 + i, &rq, &t, fault);
    nvq[i] = clamp_nvis(n_visible(t, m, n_win), kic.n_entries, r, fault,
                        c_first == 0 && threadIdx.x == 0);
    nv_max = nvq[i] > nv_max ? nvq[i] : nv_max;
  }
  const int n_active = nv_max > 0 ? (int)((nv_max + kCH - 1) / kCH) : 1;
  if (c_first >= n_active) return;
  if (c_first == 0)
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (threadIdx.x == i) ws.state[(int64_t)(q0 + i) * kStateInts + 5] = (int32_t)nvq[i];

  constexpr int NT = kCH / 4 / 16;
  typedef typename std::conditional<F8K, u32x4, bf16x8>::type KeyT;
  const int64_t cb = (int64_t)c_first * kCH;
  const int64_t w0b = cb + (int64_t)wv * (kCH / 4);
  const int64_t c_end = nv_max < cb + kCH ? nv_max : cb + kCH;
  float ksc[2];
  if constexpr (F8K) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      ksc[j] = (unsigned)pid[j] < (unsigned)kic.n_pages ? kic.scale[pid[j]] : 1.f;
  }
  KeyT x0[NT], x1[NT];
  const int r8 = lane >> 3, p8 = lane & 7;   // bf16 loads: key r8 of 8, 16-byte piece p8
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int pg = pid[u >> 2];
    const bool okp = (unsigned)pg < (unsigned)kic.n_pages;
    if constexpr (F8K) {
      // 16 whole 64-byte keys per load instruction, as in idx_scan_kernel
      x0[u] = __builtin_nontemporal_load(
          (const KeyT*)(kic.data + ((int64_t)(okp ? pg : 0) * kPage + 16 * (u & 3) + row) * kDI) + g);
    } else {
      // whole 128-byte keys, 8 per load instruction, as in idx_scan_kernel
      const KeyT* kr = (const KeyT*)(kic.data + ((int64_t)(okp ? pg : 0) * kPage +
                                                 16 * (u & 3) + r8) * (kDI * 2)) + p8;
      x0[u] = __builtin_nontemporal_load(kr);
      x1[u] = __builtin_nontemporal_load(kr + 8 * (kDI * 2 / 16));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (w0b + 64 * j < c_end && (unsigned)pid[j] >= (unsigned)kic.n_pages)
        atomicOr(fault, HSA_FAULT_PAGE);
  }
  // A rows 4i..4i+3: query i's four heads
  bf16x8 a0 = {}, a1 = {};
  if ((row >> 2) < G) {
    const bf16x8* qa = (const bf16x8*)(qI + ((int64_t)(q0 + (row >> 2)) * kHI + (row & 3)) * kDI);
    a0 = qa[F8K ? 2 * g : g];   // the keys' channel order, as in idx_scan_kernel
    a1 = qa[F8K ? 2 * g + 1 : 4 + g];
  }
  // this lane group's query: weights and visible blocks
  const bool gq = g < G;
  float wg[kHI];
#pragma unroll
  for (int h = 0; h < kHI; ++h) wg[h] = gq ? w[(int64_t)(q0 + g) * kHI + h] : 0.f;
  int64_t nv_g = 0;
#pragma unroll
  for (int i = 0; i < G; ++i)
    if (g == i) nv_g = nvq[i];
  const int64_t b_end_g = nv_g < cb + kCH ? nv_g : cb + kCH;

  __shared__ uint32_t lh2[G][kBins / 2];
  __shared__ float lsc[G][kCH];
  __shared__ bf16x8 ltile[F8K ? 1 : 4][F8K ? 1 : 128];   // bf16: one 16-key tile per wave
  for (int i = threadIdx.x; i < G * (kBins / 2); i += 256) (&lh2[0][0])[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    bf16x8 k0, k1;
    if constexpr (F8K) {
      k0 = e4m3x8_to_bf16x8(x0[u].xy);
      k1 = e4m3x8_to_bf16x8(x0[u].zw);
    } else {
      // through the wave's swizzled LDS tile into the MFMA layout, as in
      // idx_scan_kernel
      asm volatile("" ::: "memory");
      ltile[wv][r8 * 8 + (p8 ^ r8)] = x0[u];
      ltile[wv][(8 + r8) * 8 + (p8 ^ r8)] = x1[u];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      k0 = ltile[wv][row * 8 + (g ^ (row & 7))];
      k1 = ltile[wv][row * 8 + ((4 + g) ^ (row & 7))];
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, k0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, k1, acc, 0, 0, 0);
    const int64_t b = w0b + 16 * u + row;
    if (gq && b < b_end_g) {
      float sc = wg[0] * fmaxf(acc[0], 0.f) + wg[1] * fmaxf(acc[1], 0.f) +
                 wg[2] * fmaxf(acc[2], 0.f) + wg[3] * fmaxf(acc[3], 0.f);
      if constexpr (F8K) sc *= ksc[u >> 2];
      lsc[g][b - cb] = sc;
      const uint32_t bin = order_key(sc) >> 20;
      atomicAdd(&lh2[g][bin >> 1], 1u << ((bin & 1) * 16));
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float* srow = ws.scores + (int64_t)(q0 + i) * ws.R;
    const int64_t e = nvq[i] < cb + kCH ? nvq[i] : cb + kCH;
    for (int j = threadIdx.x; j < kCH; j += 256)
      if (cb + j < e) srow[cb + j] = lsc[i][j];
  }
#pragma unroll
  for (int i = 0; i < G; ++i) write_hist_list16(&lh2[i][0], ws, q0 + i, blockIdx.x);
}

// ---------------------------------------------------------------- prefill: score GEMM

// 16 consecutive query tokens per workgroup (4 A tiles of 4 queries x 4 heads,
// gridDim.y), blocks split over gridDim.x; every wave walks 16-block B tiles.
// The block range is the fast grid index and the number of ranges a multiple
// of 8: workgroups are dealt to the 8 XCDs round-robin, so each XCD's L2
// holds the keys of one eighth of the blocks instead of all of them.
template <bool F8K, bool F4K, bool S16>
__global__ __launch_bounds__(256) void idx_gemm_kernel(Queries Q, int q_base, int nq,
                                                       const u16* __restrict__ qI,
                                                       const float* __restrict__ w, Paged kic,
                                                       int m, int n_win, IdxWs ws, int* fault) {
  const int qt = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, row = lane & 15, g = lane >> 4;
  const int r8 = lane >> 3, p8 = lane & 7;   // bf16 loads: key r8 of 8, 16-byte piece p8
  const int r = Q.span_req;
  const int64_t ne = kic.n_entries[r];
  bf16x8 a[4][2];
  float wq[4][4];
  int64_t nvq[4];
  int64_t nv_max = 0;
#pragma unroll
  for (int at = 0; at < 4; ++at) {
    int ql = 16 * qt + 4 * at + (row >> 2);      // local row of the A operand's query
    a[at][0] = bf16x8{};
    a[at][1] = bf16x8{};
    if (!F4K && ql < nq) {   // (fp4: the queries are quantized into LDS below)
      const bf16x8* qa =
          (const bf16x8*)(qI + ((int64_t)(q_base + ql) * kHI + (row & 3)) * kDI);
      a[at][0] = qa[g];
      a[at][1] = qa[4 + g];
    }
    int qg = 16 * qt + 4 * at + g;               // local query of this lane's result rows
    nvq[at] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[at][i] = 0.f;
    if (qg < nq) {
      int64_t t = Q.span_pos0 + q_base + qg;
      int64_t nv = n_visible(t, m, n_win);
      nvq[at] = nv < ne ? nv : ne;
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[at][i] = w[(int64_t)(q_base + qg) * kHI + i];
    }
  }
  // every query's visible blocks (clamped to the cache), for the selection
  if (blockIdx.x == 0 && wv == 0 && row == 0) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      const int qg = 16 * qt + 4 * at + g;
      if (qg < nq) ws.state[(int64_t)qg * kStateInts + 5] = (int32_t)nvq[at];
    }
  }
  {
    int ql = 16 * qt + 15 < nq ? 16 * qt + 15 : nq - 1;
    int64_t nv = n_visible(Q.span_pos0 + q_base + ql, m, n_win);
    if (nv > ne) {
      if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(fault, HSA_FAULT_ENTRIES);
      nv = ne;
    }
    nv_max = nv;
  }
  const int64_t n_tiles = (nv_max + 15) / 16;
  const int64_t per = (n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t t_lo = per * blockIdx.x;
  const int64_t t_hi = t_lo + per < n_tiles ? t_lo + per : n_tiles;
  // physical pages of the workgroup's tile range, resolved once
  __shared__ int pg[kGemmMaxPages];
  const int64_t p_lo = (16 * t_lo) >> 6;
  const int64_t n_pg = t_hi > t_lo ? (((16 * t_hi - 1) >> 6) + 1 - p_lo) : 0;
  const bool pg_lds = n_pg <= kGemmMaxPages;
  if (pg_lds)
    for (int i = threadIdx.x; i < n_pg; i += 256)
      pg[i] = (p_lo + i) * 64 < nv_max ? kic.page_of(r, (p_lo + i) * 64, fault) : -1;
  // fp4 keys: the workgroup's 16 queries x 4 heads in MX FP4 (the indexer
  // computes in FP4), quantized once into LDS; the A operand of tile at: lane
  // (row, g < 2) holds block g of row 16 at + row (query 4 at + row / 4, head
  // row % 4), the other lanes zero codes with scale 1
  __shared__ __align__(16) uint32_t qcodes[F4K ? 64 : 1][8];
  __shared__ uint8_t qsb[F4K ? 64 : 1][2];
  if constexpr (F4K) {
    const int nql = nq - 16 * qt < 16 ? nq - 16 * qt : 16;
    mx_fp4_rows(qI + (int64_t)(q_base + 16 * qt) * kHI * kDI, 64, nql * kHI, qcodes, qsb);
  }
  __syncthreads();
  u32x4 af[F4K ? 4 : 1];
  uint32_t as[F4K ? 4 : 1];
  if constexpr (F4K) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      af[at] = u32x4{0u, 0u, 0u, 0u};
      as[at] = 127u;
      if (g < 2) {
        af[at] = *(const u32x4*)&qcodes[16 * at + row][4 * g];
        as[at] = qsb[16 * at + row][g];
      }
    }
  }
  // branch-free key loads (rows past the end, or on a bad page, read row 0 of
  // page 0 and are never stored); the next tile's keys load while this one's
  // scores are computed
  // key pieces: bf16 (16 bytes), fp8 codes (8 bytes, widened to bf16 when
  // scored, with the page scale applied to the head sum) or an fp4 MX block
  // (16 bytes; its scale byte in x1.x)
  typedef typename std::conditional<F4K, u32x4,
                                    typename std::conditional<F8K, u32x2, bf16x8>::type>::type KeyT;
  auto load = [&](int64_t tile, KeyT& x0, KeyT& x1, float& sc) {
    const int64_t b = 16 * tile + row;
    int page = -1;
    if (b < nv_max) page = pg_lds ? pg[(b >> 6) - p_lo] : kic.page_of(r, b, fault);
    const bool ok = page >= 0;
    const KeyT* kr = (const KeyT*)kic.row(ok ? page : 0, ok ? b : 0);
    if constexpr (F4K) {
      // the B operand: lane (row, g) block g & 1 of the key (lanes g >= 2 meet
      // zero query codes)
      x0 = kr[g & 1];
      const int64_t er = (int64_t)(ok ? page : 0) * kPage + (ok ? (b & 63) : 0);
      x1.x = ((const uint8_t*)kic.scale)[er * (kDI / 32) + (g & 1)];
    } else if constexpr (F8K) {
      x0 = kr[g];
      x1 = kr[4 + g];
    } else {
      // whole 128-byte keys, 8 per load instruction (lane (r8, p8): piece p8 of
      // keys r8 and r8 + 8 of the tile), as in the decode scan; a tile is 16
      // keys of one page, so its first key's page serves both loads, and keys
      // past the row's end are read but never stored
      const int64_t bt = 16 * tile;            // < nv_max for every tile walked
      const int pt = pg_lds ? pg[(bt >> 6) - p_lo] : kic.page_of(r, bt, fault);
      const KeyT* kt = (const KeyT*)(kic.data + ((int64_t)(pt >= 0 ? pt : 0) * kPage +
                                                 (bt & 63) + r8) * (kDI * 2)) + p8;
      x0 = kt[0];
      x1 = kt[8 * (kDI * 2 / 16)];
    }
    if constexpr (F8K) sc = ok ? kic.scale[page] : 1.f;
  };
  __shared__ bf16x8 ltile[F8K || F4K ? 1 : 4][F8K || F4K ? 1 : 128];   // bf16: a tile per wave
  KeyT c0, c1, n0 = {}, n1 = {};
  float cs = 1.f, ns = 1.f;
  int64_t tile = t_lo + wv;
  if (tile < t_hi) load(tile, c0, c1, cs);
  for (; tile < t_hi; tile += 4) {
    if (tile + 4 < t_hi) load(tile + 4, n0, n1, ns);
    const int64_t b = 16 * tile + row;
    bf16x8 k0, k1;
    if constexpr (F8K) {
      k0 = e4m3x8_to_bf16x8(c0);
      k1 = e4m3x8_to_bf16x8(c1);
    } else if constexpr (F4K) {
      // (scored by the MX FP4 MFMA below)
    } else {
      // through the wave's swizzled LDS tile into the MFMA layout (as the scan)
      asm volatile("" ::: "memory");
      ltile[wv][r8 * 8 + (p8 ^ r8)] = c0;
      ltile[wv][(8 + r8) * 8 + (p8 ^ r8)] = c1;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      k0 = ltile[wv][row * 8 + (g ^ (row & 7))];
      k1 = ltile[wv][row * 8 + ((4 + g) ^ (row & 7))];
    }
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F4K) {
        acc = mfma_mx_fp4(af[at], as[at], c0, c1.x, acc);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[at][0], k0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[at][1], k1, acc, 0, 0, 0);
      }
      if (b < nvq[at]) {
        float s = wq[at][0] * fmaxf(acc[0], 0.f) + wq[at][1] * fmaxf(acc[1], 0.f) +
                  wq[at][2] * fmaxf(acc[2], 0.f) + wq[at][3] * fmaxf(acc[3], 0.f);
        if constexpr (F8K) s *= cs;   // ReLU commutes with a scale > 0
        score_store<S16>(score_row<S16>(ws, 16 * qt + 4 * at + g), b, score_round<S16>(s));
      }
    }
    c0 = n0;
    c1 = n1;
    cs = ns;
  }
}

// prefill: first-level histogram over the stored scores
// Prefill: histogram of the fp32 scores of one query, kHistSpan blocks per
// workgroup (the 4096-bin LDS histogram is cleared and written out once per
// kHistSpan scores).

template <bool S16>
__global__ __launch_bounds__(256) void idx_hist_kernel(Queries Q, int q_base, const Paged kic,
                                                       int m, int n_win, int k, IdxWs ws,
                                                       int* fault) {
  const int qrow = blockIdx.y, slice = blockIdx.x;
  const int r = Q.span_req;
  int64_t t = Q.span_pos0 + q_base + qrow;
  int64_t nv = clamp_nvis(n_visible(t, m, n_win), kic.n_entries, r, fault, false);
  const int64_t b_begin = (int64_t)slice * kHistSpan;
  if (b_begin > 0 && b_begin >= nv) return;
  if (slice == 0 && threadIdx.x == 0) ws.state[(int64_t)qrow * kStateInts + 5] = (int32_t)nv;
  const int64_t b_end = nv < b_begin + kHistSpan ? nv : b_begin + kHistSpan;
  const void* srow = score_row<S16>(ws, qrow);
  constexpr int kPer = kHistSpan / 256;
  // all loads in flight before the histogram is cleared and filled
  float sc[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t b = b_begin + 256 * u + threadIdx.x;
    sc[u] = score_get<S16>(srow, b, b_end, ws.R);   // counted only below b_end
  }
  __shared__ uint32_t lhist[kBins];
  for (int i = threadIdx.x; i < kBins; i += 256) lhist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (b_begin + 256 * u + threadIdx.x < b_end) atomicAdd(&lhist[order_key(sc[u]) >> 20], 1u);
  write_hist_list(lhist, ws, qrow, slice);
}

// ---------------------------------------------------------------- select, refine, emit


// One workgroup per query: threshold bin from the histogram, one pass over the
// query's scores marking blocks above it in a bitmap and collecting the blocks
// inside it, radix refinement of those candidates (score bits, then inverted
// block id), and emission of the bitmap in ascending block order.  Bitmap and
// candidates live in LDS when they fit (dynamic shared memory sized by the
// host), else in the workspace.
// mode 0: the whole selection; mode 1: threshold only (long rows, before the
// multi-workgroup select kernel); mode 2: refine + emit only (after it); mode
// 3: the whole selection with the query's histogram built from its own score
// row instead of histogram lists (prefill: the scores are read from HBM once
// and again from L2, and no histogram kernel runs).
template <int NT, bool S16>
__global__ __launch_bounds__(NT) void idx_topk_kernel(int k, IdxWs ws, int32_t* __restrict__ idx,
                                                      float* __restrict__ score, int out_row0,
                                                      int cand_lds, int bm_lds_words, int mode) {
  constexpr int BPT = kBins / NT;                // histogram bins per thread
  extern __shared__ __align__(16) uint64_t dyn[];
  __shared__ uint32_t sh[NT / 64];
  __shared__ int s_thr, s_above, s_dstar;
  __shared__ uint32_t s_ncand, s_next, s_dabove;
  __shared__ uint32_t h256[256];
  __shared__ uint64_t sh64[S16 ? 2 * (NT / 64) : 1];
  const int qrow = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* st = ws.state + (int64_t)qrow * kStateInts;
  const int64_t nv = st[5];
  const void* srow = score_row<S16>(ws, qrow);

  // first round of scores, loaded before the threshold search (independent of
  // it).  bf16 rows keep the raw 16 bits until the scores are classified: a
  // conversion here would make the threshold search wait for these loads.
  constexpr int U = NT >= 1024 ? 32 : 16;
  float sc0[U];
  uint32_t raw0[S16 ? U : 1];
  const bool whole = mode == 0 || mode == 3;
  if (whole) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = (int64_t)u * NT + tid;
      if constexpr (S16)
        raw0[u] = ((const u16*)srow)[b < ws.R ? b : ws.R - 1];
      else
        sc0[u] = b < ws.R ? ((const float*)srow)[b] : 0.f;
    }
  }
  // mode 2: the threshold state, the first NT chunk candidate counts and the
  // bitmap (into LDS when the host sized it in) are requested together, so
  // the kernel waits for one round trip before the candidates
  uint32_t cnt0 = 0;
  uint32_t* bm_l = (uint32_t*)(dyn + 2 * (int64_t)cand_lds);
  if (mode == 2) {
    const int thr2 = st[2], above2 = st[3], dab2 = st[6];
    const int n_ch = (int)(ws.R / kSelCH);
    if (tid < n_ch) cnt0 = (uint32_t)ws.ccount[(int64_t)qrow * n_ch + tid];
    const int W4 = bm_lds_words / 4;
    const uint4* bsrc = (const uint4*)(ws.bitmap + (int64_t)qrow * (ws.R / 32));
    if constexpr (NT >= 1024) {
      constexpr int kBmPer = kBmLdsMaxWords / 4 / NT;
      uint4 bw[kBmPer];
#pragma unroll
      for (int u = 0; u < kBmPer; ++u)
        if (u * NT + tid < W4) bw[u] = bsrc[u * NT + tid];
#pragma unroll
      for (int u = 0; u < kBmPer; ++u)
        if (u * NT + tid < W4) ((uint4*)bm_l)[u * NT + tid] = bw[u];
    } else {
      for (int i = tid; i < W4; i += NT) ((uint4*)bm_l)[i] = bsrc[i];
    }
    if (tid == 0) { s_thr = thr2; s_above = above2; s_dabove = dab2; }
    __syncthreads();
  } else {
  // ---- threshold bin: thread i owns bins kBins-BPT(i+1) .. kBins-BPT*i-1 (descending)
  if (tid == 0) { s_thr = -1; s_above = 0; s_ncand = 0; }
  {
    // the query's histogram, merged in LDS from its lists (the dynamic LDS is
    // free until candidates are collected).  Each wave takes LB lists at a
    // time and loads their first 128 entries together, counts included, so a
    // step costs one memory round trip; entries past a list's count are
    // ignored.
    uint32_t* lh = (uint32_t*)dyn;
    if (mode == 3) {
      // the row's own histogram: the first round from the scores already
      // loaded, the rest in rounds of U loads per thread
      for (int i = tid; i < kBins; i += NT) lh[i] = 0;
      __syncthreads();
      for (int64_t base = 0; base < nv; base += (int64_t)NT * U) {
        float hv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t b = base + (int64_t)u * NT + tid;
          float s0;
          if constexpr (S16) s0 = __uint_as_float(raw0[u] << 16);
          else s0 = sc0[u];
          hv[u] = base == 0 ? s0 : score_get<S16>(srow, b, nv, ws.R);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (base + (int64_t)u * NT + tid < nv) atomicAdd(&lh[order_key(hv[u]) >> 20], 1u);
      }
    } else {
    const int32_t* hn = ws.hl_n + (int64_t)qrow * ws.n_lists;
    const uint32_t* hlq = ws.hl + (int64_t)qrow * ws.n_lists * ws.list_cap;
    constexpr int NWV = NT / 64, LB = 8;
    int cnt[LB];
    uint32_t e0[LB], e1[LB];
    // lists c0 .. c0 + LB - 1, clamped to the workspace's lists; the counts of
    // lists past the row's visible blocks are dropped once its length is known
    auto load_step = [&](int c0) {
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int c = c0 + j < ws.n_lists ? c0 + j : ws.n_lists - 1;
        cnt[j] = hn[c];
        const uint32_t* L = hlq + (int64_t)c * ws.list_cap;   // list_cap >= 128
        e0[j] = L[lane];
        e1[j] = L[64 + lane];
      }
    };
    // the first step's lists are requested before the row length arrives and
    // while the LDS histogram is cleared
    if (wv * LB < ws.n_lists) load_step(wv * LB);
    for (int i = tid; i < kBins; i += NT) lh[i] = 0;
    __syncthreads();
    const int n_used = nv > 0 ? (int)((nv + ws.list_span - 1) / ws.list_span) : 1;
    for (int c0 = wv * LB; c0 < n_used; c0 += NWV * LB) {
      if (c0 != wv * LB) load_step(c0);
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int nj = c0 + j < n_used ? cnt[j] : 0;
        if (lane < nj) atomicAdd(&lh[e0[j] >> 16], e0[j] & 0xFFFFu);
        if (64 + lane < nj) atomicAdd(&lh[e1[j] >> 16], e1[j] & 0xFFFFu);
        for (int i = 128 + lane; i < nj; i += 64) {   // long lists
          const uint32_t e = hlq[(int64_t)(c0 + j) * ws.list_cap + i];
          atomicAdd(&lh[e >> 16], e & 0xFFFFu);
        }
      }
    }
    }
    __syncthreads();
    uint32_t v[BPT];
    const int lo = kBins - BPT * (tid + 1);
#pragma unroll
    for (int j = 0; j < BPT; ++j) v[j] = lh[lo + j];
    uint32_t sm = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) sm += v[j];
    uint32_t tot;
    const uint32_t pre = block_scan_nt<NT>(sm, &tot, sh);
    if (nv > k && pre < (uint32_t)k && pre + sm >= (uint32_t)k) {
      uint32_t cum = pre;
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (cum < (uint32_t)k && cum + v[j] >= (uint32_t)k) {
          s_thr = lo + j;
          s_above = (int)cum;
          s_dabove = v[j];            // candidates in the threshold bin
        }
        cum += v[j];
      }
    }
  }
  __syncthreads();
  if (mode == 1) {
    if (tid == 0) { st[2] = s_thr; st[3] = s_above; st[6] = s_thr >= 0 ? (int)s_dabove : 0; }
    return;
  }
  }
  const int thr = s_thr;
  const uint32_t n_thr_bin = thr >= 0 ? s_dabove : 0;
  uint64_t* ca = dyn;
  uint64_t* cb = dyn + cand_lds;
  const int64_t W = (nv + 31) / 32;
  const bool cand_in_lds = n_thr_bin <= (uint32_t)cand_lds;
  uint64_t* csrc = cand_in_lds ? ca : ws.cand + (int64_t)qrow * ws.R;
  uint64_t* cdst = cand_in_lds ? cb : ws.cand2 + (int64_t)qrow * ws.R;
  if (mode == 2) {
    // candidates sit in per-chunk regions of cand (chunk c at c*kSelCH, ccount[c]
    // of them): compact them into LDS, or into cand2 when they do not fit
    const int n_ch = (int)(ws.R / kSelCH);
    const int32_t* cc = ws.ccount + (int64_t)qrow * n_ch;
    const uint64_t* g = ws.cand + (int64_t)qrow * ws.R;
    uint64_t* dstc = cand_in_lds ? ca : ws.cand2 + (int64_t)qrow * ws.R;
    // chunk offsets by a block scan, then every thread copies whole candidates:
    // candidate i lies in the chunk c with off[c] <= i < off[c + 1]
    __shared__ uint32_t coff[kMaxSelChunks + 1];
    uint32_t run = 0;
    for (int c0 = 0; c0 < n_ch; c0 += NT) {
      const int c = c0 + tid;
      const uint32_t cnt = c0 == 0 ? cnt0 : (c < n_ch ? (uint32_t)cc[c] : 0u);
      uint32_t tot;
      const uint32_t off = block_scan_nt<NT>(cnt, &tot, sh) + run;
      if (n_ch <= kMaxSelChunks) {
        if (c < n_ch) coff[c] = off;
      } else {
        for (uint32_t i = 0; i < cnt; ++i) dstc[off + i] = g[(int64_t)c * kSelCH + i];
      }
      run += tot;
      __syncthreads();   // sh is reused by the next round's scan
    }
    if (n_ch <= kMaxSelChunks) {
      if (tid == 0) coff[n_ch] = run;
      __syncthreads();
      for (uint32_t i = tid; i < run; i += NT) {
        int lo = 0, hi = n_ch;        // coff[lo] <= i < coff[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (coff[mid] <= i) lo = mid; else hi = mid;
        }
        dstc[i] = g[(int64_t)lo * kSelCH + (i - coff[lo])];
      }
    }
    if (tid == 0) s_ncand = run;
    __threadfence_block();
    __syncthreads();
    csrc = dstc;
    cdst = cand_in_lds ? cb : ws.cand + (int64_t)qrow * ws.R;
  }
  const bool bm_in_lds = W <= bm_lds_words;
  uint32_t* bm = bm_in_lds ? bm_l : ws.bitmap + (int64_t)qrow * (ws.R / 32);

  // ---- one pass over the scores: bitmap of blocks above the bin, candidates in it
  for (int64_t base = 0; whole && base < nv; base += (int64_t)NT * U) {
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = base + (int64_t)u * NT + tid;
      float s0;
      if constexpr (S16) s0 = __uint_as_float(raw0[u] << 16);
      else s0 = sc0[u];
      sc[u] = base == 0 ? s0 : score_get<S16>(srow, b, nv, ws.R);   // classified below nv
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b0 = base + (int64_t)u * NT;
      if (b0 >= nv) break;
      const int64_t b = b0 + tid;
      const bool valid = b < nv;
      const uint32_t key = order_key(sc[u]);
      const int bin = (int)(key >> 20);
      const bool sel = valid && (thr < 0 || bin > thr);
      const bool cnd = valid && thr >= 0 && bin == thr;
      const uint64_t cmask = __ballot(cnd);
      if (cmask) {
        const int leader = __ffsll((unsigned long long)cmask) - 1;
        uint32_t cbase = 0;
        if (lane == leader) cbase = atomicAdd(&s_ncand, (uint32_t)__popcll(cmask));
        cbase = __shfl(cbase, leader);
        if (cnd) csrc[cbase + __popcll(cmask & ((1ull << lane) - 1))] =
                     ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)b);
      }
      const uint64_t mask = __ballot(sel);
      const int64_t wb = b0 + 64 * wv;
      if (lane == 0 && wb < nv) {
        bm[wb >> 5] = (uint32_t)mask;
        if (wb + 32 < nv) bm[(wb >> 5) + 1] = (uint32_t)(mask >> 32);
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // ---- refine the threshold bin: need = k - (count above the bin)
  if (thr >= 0) {
    int need = k - s_above;
    uint32_t nc = s_ncand;
    int shift = 44;   // bits 63..52 of the composite key were the histogram bin
    // at most 7 digit passes cover the remaining 52 key bits (scores, then ids);
    // keys are unique (they contain the block id), so the candidates left after
    // the last pass are exactly the ones still needed.  fp32 scores take the
    // 8-bit digits in turn (they rarely tie, so one or two passes end it).
    // bf16 scores tie often: a pass there takes the 8 bits from the highest
    // bit in which the candidates still differ (an AND / OR reduction finds
    // it), so no pass is spent on bits they all share; the candidates left
    // share every bit down to that digit, so the next pass starts at least 8
    // bits lower and 7 passes still suffice.
    for (int pass = 0; need > 0; ++pass, shift -= 8) {
      if (nc <= (uint32_t)need || pass >= 7) {
        for (uint32_t i = tid; i < nc; i += NT) {
          const uint32_t b = ~(uint32_t)ld_cand(csrc + i);
          atomicOr(bm + (b >> 5), 1u << (b & 31));
        }
        break;
      }
      uint64_t dmask = shift >= 0 ? 0xFFull : 0xFull;
      int sh_amt = shift >= 0 ? shift : 0;
      if constexpr (S16) {
        uint64_t ka = ~0ull, ko = 0;
        for (uint32_t i = tid; i < nc; i += NT) {
          const uint64_t x = ld_cand(csrc + i);
          ka &= x;
          ko |= x;
        }
        block_and_or<NT>(&ka, &ko, sh64);
        if (ka == ko) break;   // identical keys cannot occur: stop rather than loop
        const int top = 63 - __clzll(ka ^ ko);
        sh_amt = top >= 7 ? top - 7 : 0;
        dmask = 0xFFull;
      }
      if (tid < 256) h256[tid] = 0;
      if (tid == 0) { s_next = 0; s_dstar = -1; }
      __syncthreads();
      for (uint32_t i = tid; i < nc; i += NT)
        atomicAdd(&h256[(ld_cand(csrc + i) >> sh_amt) & dmask], 1u);
      __syncthreads();
      {
        // digit crossing by a block scan (threads >= 256 carry zeros)
        const uint32_t c = tid < 256 ? h256[255 - tid] : 0u;
        uint32_t tot;
        const uint32_t pre = block_scan_nt<NT>(c, &tot, sh);
        if (tid < 256 && pre < (uint32_t)need && pre + c >= (uint32_t)need) {
          s_dstar = 255 - tid;
          s_dabove = pre;
        }
      }
      __syncthreads();
      const int dstar = s_dstar;
      if (dstar < 0) break;   // counts inconsistent: stop rather than loop
      for (uint32_t i = tid; i < nc; i += NT) {
        const uint64_t key = ld_cand(csrc + i);
        const int dg = (int)((key >> sh_amt) & dmask);
        if (dg > dstar) {
          const uint32_t b = ~(uint32_t)key;
          atomicOr(bm + (b >> 5), 1u << (b & 31));
        } else if (dg == dstar) {
          cdst[atomicAdd(&s_next, 1u)] = key;
        }
      }
      __threadfence_block();
      __syncthreads();
      need -= (int)s_dabove;
      nc = s_next;
      uint64_t* tmp = csrc; csrc = cdst; cdst = tmp;
      __syncthreads();
    }
  }
  __threadfence_block();
  __syncthreads();

  // ---- emit ascending block ids: each thread owns wpt consecutive bitmap
  // words per round (loaded together; wpt = 8 on long rows, fewer on short
  // ones so that a dense bitmap's bits spread over more threads); a block scan
  // of their popcounts gives its output offset
  int32_t* irow = idx + (int64_t)(out_row0 + qrow) * k;
  float* srow_out = score ? score + (int64_t)(out_row0 + qrow) * k : nullptr;
  uint32_t total = 0;
  const int wpt = W >= (int64_t)NT * 8 ? 8 : (int)((W + NT - 1) / NT);
  for (int64_t r0 = 0; r0 < W; r0 += (int64_t)NT * wpt) {
    const int64_t w0 = r0 + (int64_t)tid * wpt;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wd[i] = i < wpt && w0 + i < W ? (bm_in_lds ? bm_l[w0 + i] : ld_agent(bm + w0 + i)) : 0u;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += __popc(wd[i]);
    uint32_t tot;
    uint32_t o = block_scan_nt<NT>(cnt, &tot, sh) + total;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = wd[i];
      while (word) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        const uint32_t b = (uint32_t)((w0 + i) * 32 + bit);
        if (o < (uint32_t)k) {
          irow[o] = (int32_t)b;
          if (srow_out) srow_out[o] = score_load<S16>(srow, b);
        }
        ++o;
      }
    }
    total += tot;
    __syncthreads();   // sh is reused by the next round's scan
  }
  for (int i = (int)total + tid; i < k; i += NT) {
    irow[i] = -1;
    if (srow_out) srow_out[i] = 0.f;
  }
  if (tid < kStateInts) st[tid] = 0;
}

// Long rows: mark the blocks of one 2048-block chunk above the threshold bin
// (found by idx_topk_kernel mode 1) and append the ones inside it.
template <bool S16>
__global__ __launch_bounds__(256) void idx_select_kernel(IdxWs ws) {
  const int qrow = blockIdx.y, chunk = blockIdx.x;
  int32_t* st = ws.state + (int64_t)qrow * kStateInts;
  const void* srow = score_row<S16>(ws, qrow);
  const int64_t b_begin = (int64_t)chunk * kSelCH;
  constexpr int kPer = kSelCH / 256;
  float sc[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) sc[u] = score_load<S16>(srow, b_begin + 256 * u + threadIdx.x);   // within R
  const int64_t nv = st[5];
  const int thr = st[2];
  uint32_t* bm = ws.bitmap + (int64_t)qrow * (ws.R / 32);
  uint64_t* cand = ws.cand + (int64_t)qrow * ws.R + b_begin;   // this chunk's region
  __shared__ uint32_t s_cnt;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t b_end = nv < b_begin + kSelCH ? nv : b_begin + kSelCH;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t base = b_begin + 256 * u;
    const int64_t b = base + threadIdx.x;
    const bool valid = b < b_end;
    const uint32_t key = order_key(sc[u]);
    const int bin = (int)(key >> 20);
    const bool sel = valid && (thr < 0 || bin > thr);
    const bool cnd = valid && thr >= 0 && bin == thr;
    const uint64_t cmask = __ballot(cnd);
    if (cmask) {
      const int leader = __ffsll((unsigned long long)cmask) - 1;
      uint32_t cbase = 0;
      if (lane == leader) cbase = atomicAdd(&s_cnt, (uint32_t)__popcll(cmask));
      cbase = __shfl(cbase, leader);
      if (cnd)
        cand[cbase + __popcll(cmask & ((1ull << lane) - 1))] =
            ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)b);
    }
    const uint64_t mask = __ballot(sel);
    const int64_t wb = base + 64 * wv;
    if (lane == 0 && wb < b_end) {
      bm[wb >> 5] = (uint32_t)mask;
      if (wb + 32 < b_end) bm[(wb >> 5) + 1] = (uint32_t)(mask >> 32);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) ws.ccount[(int64_t)qrow * (ws.R / kSelCH) + chunk] = (int32_t)s_cnt;
}

// The k-th largest of n unique 64-bit keys key(i), i < n, all sharing the bits
// above bit `bits` with `prefix`: radix digits of up to 8 bits from bit bits-1
// down (every thread of the NT-thread workgroup calls it; h256 and sh are
// workgroup scratch).  Stops as soon as the keys sharing the digits chosen so
// far are exactly the ones still needed, so the returned threshold T
// satisfies: key >= T  <=>  key is among the k largest.
template <int NT, typename KeyFn>
__device__ uint64_t radix_kth(int64_t n, int k, KeyFn key, int bits, uint64_t prefix,
                              uint32_t* h256, uint32_t* sh) {
  __shared__ int s_d;
  __shared__ uint32_t s_above, s_cnt;
  uint64_t mask = bits >= 64 ? 0ull : ~0ull << bits;
  uint32_t need = (uint32_t)k;
  for (int hi = bits; hi > 0; hi -= 8) {
    const int wdt = hi >= 8 ? 8 : hi, shift = hi - wdt;
    const uint64_t dm = (1ull << wdt) - 1;
    if (threadIdx.x < 256) h256[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += NT) {
      const uint64_t x = key(i);
      if ((x & mask) == prefix) atomicAdd(&h256[(x >> shift) & dm], 1u);
    }
    __syncthreads();
    {
      const uint32_t c = threadIdx.x < 256 ? h256[255 - threadIdx.x] : 0u;
      uint32_t tot;
      const uint32_t pre = block_scan_nt<NT>(c, &tot, sh);
      if (threadIdx.x < 256 && pre < need && pre + c >= need) {
        s_d = 255 - (int)threadIdx.x;
        s_above = pre;
        s_cnt = c;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_d << shift;
    mask |= dm << shift;
    need -= s_above;
    const uint32_t cnt = s_cnt;
    __syncthreads();   // s_d, s_above, s_cnt are rewritten by the next digit
    if (cnt == need) break;   // all keys with this prefix are selected
  }
  return prefix;
}

// Decode, long rows: the top-k of a query from the candidates its scan
// workgroups wrote.  With T the k-th largest candidate key, the union holds the
// row's top-k exactly when T's bin is at least every workgroup's cut bin (all
// scores left out lie below that bin, so below T); otherwise (or when a
// workgroup overflowed its candidate space) the k-th key is selected over the
// whole score row.  The selected ids are marked in an LDS bitmap and emitted
// ascending.  One workgroup per query.
// Workgroups past the queries (blockIdx.x >= n_q) run the decode cache upkeep
// of request blockIdx.x - n_q, fp8 caches included: the selection reads no
// cache, and the attention that reads them is the next launch.
// (one 1024-thread workgroup per CU is all it needs: four waves per SIMD, so
// the registers of four, and no spill of the many scalar arguments to memory)
template <bool S16>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4))) void idx_cand_kernel(int k, IdxWs ws, int32_t* __restrict__ idx,
                                                        float* __restrict__ score, int n_q,
                                                        UpdateArgs upd, int* fault) {
  constexpr int NT = 1024, BPT = kBins / NT;
  constexpr int TB = kTopBins * kCandMaxLists / NT;   // top-bin slots a thread loads
  constexpr int SPEC = 8;                              // candidates a thread loads up front
  if ((int)blockIdx.x >= n_q) {
    decode_update_body<true>(upd, blockIdx.x - n_q, fault);
    return;
  }
  extern __shared__ __align__(16) uint64_t dyn[];
  uint64_t* tc = dyn;                                     // [kThrCandMax] threshold-bin candidates
  uint32_t* bm = (uint32_t*)(dyn + kThrCandMax);          // [R / 32]
  __shared__ uint32_t sh[NT / 64];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t hist[kBins];
  __shared__ int16_t s_cnt[kCandMaxLists];               // candidates of each live list
  __shared__ uint8_t s_ntop[kCandMaxLists];              // top bins of each live list
  __shared__ int s_bad, s_maxbc, s_thr, s_ovf;
  __shared__ uint32_t s_above, s_ntc, s_tot;
  const int qrow = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  int32_t* st = ws.state + (int64_t)qrow * kStateInts;
  const void* srow = score_row<S16>(ws, qrow);
  int32_t* irow = idx + (int64_t)qrow * k;
  float* srow_out = score ? score + (int64_t)qrow * k : nullptr;
  // ---- every load the selection needs is issued before any is used: the
  // row length, each scan workgroup's count, cut bin, top-bin count and top
  // bins, and the first cov candidates of every list (tpl threads per list,
  // SPEC keys each; only a tie storm makes a list longer, read in a second
  // pass).  Lists past the row's own (a shorter row in the batch) are masked
  // once its length is known.
  const int nl = ws.n_lists;
  const int64_t wrow = (int64_t)qrow * nl;
  // (every load below is unconditional, from a clamped in-bounds address;
  // what lies outside a list or past its count is masked where it is used --
  // a conditional load's zero would overwrite a register still being loaded
  // and make the compiler wait for the earlier loads)
  const int tl = tid < nl ? tid : nl - 1;
  const int cnt = ws.wcnt[wrow + tl];
  const int bcw = ws.wbin[wrow + tl];
  const int ntop = ws.wntop[wrow + tl];
  uint32_t e[TB];
#pragma unroll
  for (int r = 0; r < TB; ++r) {
    const int slot = r * NT + tid, last = nl * kTopBins - 1;
    e[r] = ws.wtop[wrow * kTopBins + (slot < last ? slot : last)];
  }
  const int tpl = NT / nl;                                // threads per list (>= 4)
  const int lg = tid / tpl, sub = tid - lg * tpl;
  const int cov = tpl * SPEC < kCandCap ? tpl * SPEC : kCandCap;
  const int lgc = lg < nl ? lg : nl - 1;
  uint64_t xs[SPEC];
#pragma unroll
  for (int u = 0; u < SPEC; u += 2) {
    const int j = sub * SPEC + u < kCandCap - 2 ? sub * SPEC + u : kCandCap - 2;
    const uint4 v = *(const uint4*)(ws.wcand + (wrow + lgc) * kCandCap + j);
    xs[u] = ((uint64_t)v.y << 32) | v.x;
    xs[u + 1] = ((uint64_t)v.w << 32) | v.z;
  }
  // the row length last: the compiler waits for it at once (a uniform value),
  // and loads complete in order, so that one wait covers all of them
  const int64_t nv = st[5];
  const int64_t W = (nv + 31) / 32;
  for (int64_t i = tid; i < W; i += NT) bm[i] = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) hist[tid + NT * j] = 0;
  if (tid == 0) {
    s_bad = 0; s_maxbc = -1; s_thr = -1; s_ovf = 0; s_above = 0; s_ntc = 0; s_tot = 0;
  }
  // the loads above stay where they are: the compiler would otherwise sink
  // them to their first use, a round trip per phase
#pragma unroll
  for (int r = 0; r < TB; ++r) asm volatile("" ::"v"(e[r]));
#pragma unroll
  for (int u = 0; u < SPEC; ++u) asm volatile("" ::"v"(xs[u]));
  const int n_wg = (int)((nv + ws.list_span - 1) / ws.list_span);   // this row's lists
  int path = 0;
  if (tid < nl) {
    const bool live = tid < n_wg;
    s_cnt[tid] = (int16_t)(live ? (cnt < kCandCap ? cnt : kCandCap) : 0);
    s_ntop[tid] = (uint8_t)(live ? (ntop < kTopBins ? ntop : kTopBins) : 0);
  }
  __syncthreads();
  uint32_t tot = 0;
  if (nv > k) {
    {   // the live lists' flags, largest cut and sum: one atomic per wave
      const bool live = tid < nl && tid < n_wg;
      const bool bad = live && (cnt > kCandCap || ntop > kTopBins), ovf = live && cnt > cov;
      const int mbc = wave_max_i32(live ? bcw : -1);
      const uint32_t sum = wave_sum_u32(live ? (uint32_t)cnt : 0u);
      const uint64_t bb = __ballot(bad), bo = __ballot(ovf);
      if (lane == 0 && tid < nl) {
        if (bb) atomicOr(&s_bad, 1);
        if (bo) atomicOr(&s_ovf, 1);
        if (mbc >= 0) atomicMax(&s_maxbc, mbc);
        atomicAdd(&s_tot, sum);
      }
    }
    // the union's histogram from the workgroups' top-bin lists
#pragma unroll
    for (int r = 0; r < TB; ++r) {
      const int slot = r * NT + tid, g = slot / kTopBins, j = slot % kTopBins;
      if (g < nl && j < s_ntop[g] && e[r] != 0u) atomicAdd(&hist[e[r] >> 16], e[r] & 0xFFFFu);
    }
    __syncthreads();
    // threshold bin of the histogram in `hist` (the bin holding the k-th
    // largest key, and the count above it): thread t owns bins
    // kBins - BPT(t+1) .. kBins - BPT t - 1
    auto find_threshold = [&]() {
      const int lo = kBins - BPT * (tid + 1);
      uint32_t v[BPT], sm = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        v[j] = hist[lo + j];
        sm += v[j];
      }
      uint32_t ht;
      const uint32_t pre = block_scan_nt<NT>(sm, &ht, sh);
      if (pre < (uint32_t)k && pre + sm >= (uint32_t)k) {
        uint32_t cum = pre;
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
          if (cum < (uint32_t)k && cum + v[j] >= (uint32_t)k) { s_thr = lo + j; s_above = cum; }
          cum += v[j];
        }
      }
      __syncthreads();
    };
    // a key (score key << 32 | ~block) above the threshold bin -> bitmap; in
    // it -> the threshold-bin candidates (one slot reservation per wave)
    auto classify_thr = [&](uint64_t x, bool valid, int thr) {
      const int bin = valid ? (int)(x >> 52) : -1;
      if (bin > thr) {
        const uint32_t blk = ~(uint32_t)x;
        atomicOr(&bm[blk >> 5], 1u << (blk & 31));
      }
      const bool c = bin == thr;
      const uint64_t cm = __ballot(c);
      if (cm) {
        const int leader = __ffsll((unsigned long long)cm) - 1;
        uint32_t cb = 0;
        if (lane == leader) cb = atomicAdd(&s_ntc, (uint32_t)__popcll(cm));
        cb = lane_value(cb, leader);
        const uint32_t p = cb + __popcll(cm & ((1ull << lane) - 1));
        if (c && p < (uint32_t)kThrCandMax) tc[p] = x;
      }
    };
    find_threshold();
    // the union holds the row's top-k iff every score left out lies in a bin
    // below the threshold bin
    tot = s_tot;
    bool full = s_bad != 0 || s_thr < 0 || s_thr < s_maxbc;
    if (!full) {
      const int thr = s_thr;
      // above the bin -> bitmap; in it -> the threshold-bin candidates
      auto classify = [&](uint64_t x, bool valid) {
        const int bin = valid ? (int)(x >> 52) : -1;
        if (bin > thr) {
          const uint32_t blk = ~(uint32_t)x;
          atomicOr(&bm[blk >> 5], 1u << (blk & 31));
        }
        const bool c = bin == thr;
        const uint64_t cm = __ballot(c);
        if (cm) {
          const int leader = __ffsll((unsigned long long)cm) - 1;
          uint32_t cb = 0;
          if (lane == leader) cb = atomicAdd(&s_ntc, (uint32_t)__popcll(cm));
          cb = lane_value(cb, leader);
          const uint32_t p = cb + __popcll(cm & ((1ull << lane) - 1));
          if (c && p < (uint32_t)kThrCandMax) tc[p] = x;
        }
      };
      const int my_cnt = lg < nl ? s_cnt[lg] : 0;
      {
        // the candidates read up front: bitmap marks, then one LDS atomic per
        // wave reserves the threshold-bin slots of all of them (one
        // reservation per candidate is a dependent LDS round trip each)
        bool cin[SPEC];
        uint64_t cmk[SPEC];
        uint32_t nin = 0;
#pragma unroll
        for (int u = 0; u < SPEC; ++u) {
          const int j = sub * SPEC + u;
          const int bin = j < my_cnt && j < cov ? (int)(xs[u] >> 52) : -1;
          if (bin > thr) {
            const uint32_t blk = ~(uint32_t)xs[u];
            atomicOr(&bm[blk >> 5], 1u << (blk & 31));
          }
          cin[u] = bin == thr;
          cmk[u] = __ballot(cin[u]);
          nin += (uint32_t)__popcll(cmk[u]);
        }
        if (nin) {   // uniform in the wave
          uint32_t cb = 0;
          if (lane == 0) cb = atomicAdd(&s_ntc, nin);
          cb = lane_value(cb, 0);
          const uint64_t below = (1ull << lane) - 1;
#pragma unroll
          for (int u = 0; u < SPEC; ++u) {
            const uint32_t p = cb + (uint32_t)__popcll(cmk[u] & below);
            if (cin[u] && p < (uint32_t)kThrCandMax) tc[p] = xs[u];
            cb += (uint32_t)__popcll(cmk[u]);
          }
        }
      }
      if (s_ovf) {   // uniform: some list holds more than was read up front
        for (int base = cov; base < kCandCap; base += tpl * SPEC) {
          uint64_t y[SPEC];
#pragma unroll
          for (int u = 0; u < SPEC; ++u) {
            const int j = base + sub * SPEC + u;
            y[u] = j < my_cnt ? ws.wcand[(wrow + lg) * kCandCap + j] : 0ull;
          }
#pragma unroll
          for (int u = 0; u < SPEC; ++u) classify(y[u], base + sub * SPEC + u < my_cnt);
        }
      }
      __syncthreads();
      const uint32_t ntc = s_ntc;
      if (ntc > (uint32_t)kThrCandMax) {
        full = true;                          // uniform: every thread read s_ntc
        for (int64_t i = tid; i < W; i += NT) bm[i] = 0;
        __syncthreads();
      } else {
        const uint64_t T = radix_kth<NT>((int64_t)ntc, k - (int)s_above,
                                         [&](int64_t i) { return tc[i]; }, 52,
                                         (uint64_t)thr << 52, h256, sh);
        for (uint32_t i = tid; i < ntc; i += NT)
          if (tc[i] >= T) {
            const uint32_t blk = ~(uint32_t)tc[i];
            atomicOr(&bm[blk >> 5], 1u << (blk & 31));
          }
      }
    }
    if (tid == 0)   // which path served the query (stored at the end, off the critical path)
      path = full ? (s_bad ? 1 : (s_thr < 0 ? 2 : (s_thr < s_maxbc ? 3 : 4))) : 0;
    if (full) {
      // exact selection over the whole row: when the union cannot prove the
      // answer -- a row scanned by few workgroups (each hands over at most
      // kCandCap / 2 candidates, so under about 3k / 128 workgroups the union
      // rarely holds the top-k), a list overflow, a tie storm.  One pass builds
      // the row's histogram of the top 12 key bits and finds the threshold bin,
      // a second marks the blocks above it and collects those inside it, which
      // are refined like the union's; a threshold bin too full for LDS takes
      // the 64-bit radix selection over the row.
      auto fkey = [&](int64_t i) {
        return ((uint64_t)order_key(score_load<S16>(srow, i)) << 32) | (uint64_t)(~(uint32_t)i);
      };
#pragma unroll
      for (int j = 0; j < BPT; ++j) hist[tid + NT * j] = 0;
      for (int64_t i = tid; i < W; i += NT) bm[i] = 0;
      if (tid == 0) { s_thr = -1; s_above = 0; s_ntc = 0; }
      __syncthreads();
      for (int64_t i = tid; i < nv; i += NT)
        atomicAdd(&hist[order_key(score_load<S16>(srow, i)) >> 20], 1u);
      __syncthreads();
      find_threshold();
      const int thr = s_thr;   // (nv > k: a bin holds the k-th largest key)
      for (int64_t b0 = 0; b0 < nv; b0 += NT) {
        const int64_t i = b0 + tid;
        const bool valid = i < nv;
        classify_thr(valid ? fkey(i) : 0ull, valid, thr);
      }
      __syncthreads();
      const uint32_t ntc = s_ntc;
      if (ntc <= (uint32_t)kThrCandMax) {
        const uint64_t T = radix_kth<NT>((int64_t)ntc, k - (int)s_above,
                                         [&](int64_t i) { return tc[i]; }, 52,
                                         (uint64_t)thr << 52, h256, sh);
        for (uint32_t i = tid; i < ntc; i += NT)
          if (tc[i] >= T) {
            const uint32_t blk = ~(uint32_t)tc[i];
            atomicOr(&bm[blk >> 5], 1u << (blk & 31));
          }
      } else {
        for (int64_t i = tid; i < W; i += NT) bm[i] = 0;
        __syncthreads();
        const uint64_t T = radix_kth<NT>(nv, k, fkey, 64, 0ull, h256, sh);
        for (int64_t i = tid; i < nv; i += NT)
          if (fkey(i) >= T) atomicOr(&bm[i >> 5], 1u << (i & 31));
      }
    }
  } else {
    __syncthreads();
    for (int64_t i = tid; i < nv; i += NT) atomicOr(&bm[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  // emit ascending block ids: each thread owns 8 consecutive bitmap words per round
  uint32_t total = 0;
  for (int64_t r0 = 0; r0 < W; r0 += (int64_t)NT * 8) {
    const int64_t w0 = r0 + (int64_t)tid * 8;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wd[i] = w0 + i < W ? bm[w0 + i] : 0u;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += __popc(wd[i]);
    uint32_t tot;
    uint32_t o = block_scan_nt<NT>(cnt, &tot, sh) + total;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = wd[i];
      while (word) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        const uint32_t b = (uint32_t)((w0 + i) * 32 + bit);
        if (o < (uint32_t)k) {
          irow[o] = (int32_t)b;
          if (srow_out) srow_out[o] = score_load<S16>(srow, b);
        }
        ++o;
      }
    }
    total += tot;
    __syncthreads();   // sh is reused by the next round's scan
  }
  for (int i = (int)total + tid; i < k; i += NT) {
    irow[i] = -1;
    if (srow_out) srow_out[i] = 0.f;
  }
  if (tid == 0) {   // the path code and the union / threshold-bin sizes (diagnostics)
    st[6] = path;
    st[7] = (int32_t)((tot << 16) | (s_ntc & 0xFFFF));
  }
}

// ---------------------------------------------------------------- host launcher

// rows up to these sizes take the one-workgroup-per-query path; longer rows the
// threshold / select / refine kernels (decode: few queries, so the many-
// workgroup classification pays off earlier)
constexpr int64_t kFusedMaxBlocksDecode = 16384;
constexpr int64_t kFusedMaxBlocksPrefill = 65536;

// Top-k selection from the scores and histogram in the workspace.  Rows up to
// the fused-path size: one workgroup per query does everything (bitmap and
// candidates in LDS).  Longer rows: the threshold per query, a multi-workgroup
// pass that marks the bitmap, then one workgroup per query refines and emits.
template <bool S16>
static void launch_topk(int nt, int nq, int k, const IdxWs& ws, int32_t* idx, float* score,
                        int out_row0, hipStream_t s, bool self_hist = false) {
  const int64_t W = ws.R / 32;
  const int cand = nt == 1024 ? 2048 : 1024;
  if (ws.R <= (nt == 1024 ? kFusedMaxBlocksDecode : kFusedMaxBlocksPrefill)) {
    const int bm_words = (int)W;
    const size_t lds = (size_t)2 * cand * sizeof(uint64_t) + (size_t)bm_words * sizeof(uint32_t);
    const int mode = self_hist ? 3 : 0;
    if (nt == 1024)
      idx_topk_kernel<1024, S16><<<nq, 1024, lds, s>>>(k, ws, idx, score, out_row0, cand,
                                                       bm_words, mode);
    else
      idx_topk_kernel<256, S16><<<nq, 256, lds, s>>>(k, ws, idx, score, out_row0, cand,
                                                     bm_words, mode);
    return;
  }
  // the threshold pass merges the histogram lists in (dynamic) LDS
  idx_topk_kernel<1024, S16><<<nq, 1024, kBins * sizeof(uint32_t), s>>>(k, ws, idx, score,
                                                                         out_row0, 0, 0, 1);
  idx_select_kernel<S16><<<dim3((unsigned)(ws.R / kSelCH), nq), 256, 0, s>>>(ws);
  // the bitmap joins the candidates in LDS when it fits
  const int bm_words = W <= kBmLdsMaxWords ? (int)W : 0;
  const size_t lds = (size_t)2 * cand * sizeof(uint64_t) + (size_t)bm_words * sizeof(uint32_t);
  // rows up to 64K blocks: four waves refine and emit (cheaper barriers); longer
  // rows: sixteen (their bitmap takes 8 words per thread per round)
  if (W <= 2048)
    idx_topk_kernel<256, S16><<<nq, 256, lds, s>>>(k, ws, idx, score, out_row0, cand, bm_words,
                                                   2);
  else
    idx_topk_kernel<1024, S16><<<nq, 1024, lds, s>>>(k, ws, idx, score, out_row0, cand,
                                                     bm_words, 2);
}

hipError_t launch_indexer(const hsa_queries& q, const void* qI, const float* w,
                          const hsa_paged& kic, int m, int n_win, int k, int32_t* idx,
                          float* score, void* wsp, size_t ws_bytes, hipStream_t s,
                          const UpdateArgs* upd, int group, bool s16) {
  const bool span = q.req == nullptr && q.pos == nullptr;
  const int64_t nv_max = host_nvis(q.max_pos, m, n_win);
  const int64_t R = row_cap(nv_max);
  const unsigned n_chunks = (unsigned)(R / kCH);
  Paged kc = to_dev(kic);
  Queries Qd = to_dev(q, kic.n_req);
  int* fault = fault_word();
  if (s16 && group > 1) return hipErrorInvalidValue;   // drafts score in fp32
  // the layout this launch carves must fit the workspace it was given
  IdxWs ws;
  const int nq_ws = span ? (q.n < kSpanQC ? q.n : kSpanQC) : q.n;
  const bool grouped = !span && group > 1 && !upd;
  if (layout(nullptr, nq_ws, R, span, grouped, &ws) > ws_bytes) return hipErrorInvalidValue;
  layout((char*)wsp, nq_ws, R, span, grouped, &ws);
  if (grouped) {
    // a draft: groups of `group` queries of one request share each key pass
    const bool f8k = kic.dtype == HSA_FP8_E4M3;
    const dim3 grid(n_chunks, (unsigned)(q.n / group));
    auto scan = group == 4   ? (f8k ? idx_scan_group_kernel<4, true> : idx_scan_group_kernel<4, false>)
                : group == 3 ? (f8k ? idx_scan_group_kernel<3, true> : idx_scan_group_kernel<3, false>)
                             : (f8k ? idx_scan_group_kernel<2, true> : idx_scan_group_kernel<2, false>);
    timed_launch(HSA_K_INDEXER_SCAN, scan, grid, dim3(256), 0, s, Qd, (const u16*)qI, w, kc, m,
                 n_win, ws, fault);
    KernelTimer kt(HSA_K_INDEXER_SEL, s);
    launch_topk<false>(1024, q.n, k, ws, idx, score, 0, s);
    return hipGetLastError();
  }
  if (!span) {
    const int cpw = scan_cpw(R);
    const unsigned n_groups = (n_chunks + cpw - 1) / cpw;
    const UpdateArgs ua = upd ? *upd : UpdateArgs{};
    const bool f8k = kic.dtype == HSA_FP8_E4M3, f4k = kic.dtype == HSA_FP4_E2M1_MX;
    // eight waves, each streaming one page of every chunk
    auto pick = [&](auto k4_f8, auto k4_f4, auto k4_bf, auto k1_f8, auto k1_f4, auto k1_bf) {
      return cpw == 4 ? (f8k ? k4_f8 : f4k ? k4_f4 : k4_bf) : (f8k ? k1_f8 : f4k ? k1_f4 : k1_bf);
    };
    auto scan = s16 ? pick(idx_scan_kernel<4, 8, true, false, true>,
                           idx_scan_kernel<4, 8, false, true, true>,
                           idx_scan_kernel<4, 8, false, false, true>,
                           idx_scan_kernel<1, 8, true, false, true>,
                           idx_scan_kernel<1, 8, false, true, true>,
                           idx_scan_kernel<1, 8, false, false, true>)
                    : pick(idx_scan_kernel<4, 8, true, false, false>,
                           idx_scan_kernel<4, 8, false, true, false>,
                           idx_scan_kernel<4, 8, false, false, false>,
                           idx_scan_kernel<1, 8, true, false, false>,
                           idx_scan_kernel<1, 8, false, true, false>,
                           idx_scan_kernel<1, 8, false, false, false>);
    // long rows whose emission bitmap fits in LDS: the scan hands over
    // candidates and one kernel selects from them (two launches instead of the
    // threshold / select / refine chain)
    const bool cand = R > kFusedMaxBlocksDecode && R / 32 <= kCandBmMaxWords &&
                      ws.n_lists <= kCandMaxLists;
    // the decode cache upkeep: plain bf16 caches in the scan launch; the full
    // upkeep (fp8 page re-encoding, RoPE, fp4 indexer keys: registers the scan
    // should not carry) in the candidate selection launch, or on its own
    // before the scan
    const bool full_upd = upd && (upd->kc.dtype != HSA_BF16 || upd->vc.dtype != HSA_BF16 ||
                               upd->rope_on || (upd->csa && upd->kic.dtype != HSA_BF16));
    if (full_upd && !cand) {
      hipError_t e = launch_update(*upd, q.n, s);
      if (e != hipSuccess) return e;
    }
    const dim3 grid(n_groups + (upd && !full_upd ? 1 : 0), q.n);
    timed_launch(HSA_K_INDEXER_SCAN, scan, grid, dim3(8 * 64), 0, s, Qd, (const u16*)qI, w, kc, m,
                 n_win, k, ws, (int)n_groups, ua, cand ? k : 0, fault);
    KernelTimer kt(HSA_K_INDEXER_SEL, s);
    if (cand) {
      const size_t lds = (size_t)kThrCandMax * sizeof(uint64_t) + (size_t)(R / 32) * sizeof(uint32_t);
      const unsigned g = (unsigned)q.n + (full_upd ? (unsigned)q.n : 0u);
      if (s16)
        idx_cand_kernel<true><<<g, 1024, lds, s>>>(k, ws, idx, score, q.n, ua, fault);
      else
        idx_cand_kernel<false><<<g, 1024, lds, s>>>(k, ws, idx, score, q.n, ua, fault);
    } else if (s16) {
      launch_topk<true>(1024, q.n, k, ws, idx, score, 0, s);
    } else {
      launch_topk<false>(1024, q.n, k, ws, idx, score, 0, s);
    }
    return hipGetLastError();
  }
  const int QC = nq_ws;
  for (int q0 = 0; q0 < q.n; q0 += QC) {
    const int nq = q.n - q0 < QC ? q.n - q0 : QC;
    // chunk-local maximum of the visible blocks bounds the work of this pass
    int64_t nv_hi = host_nvis(q.span_pos0 + q0 + nq - 1, m, n_win);
    int64_t tiles = (nv_hi + 15) / 16;
    // ~128 block tiles per workgroup, in a multiple of 8 block ranges
    unsigned bsplit = (unsigned)((tiles + 127) / 128);
    if (bsplit < 1) bsplit = 1;
    if (bsplit > 512) bsplit = 512;
    bsplit = (bsplit + 7) / 8 * 8;
    const bool f8k = kic.dtype == HSA_FP8_E4M3, f4k = kic.dtype == HSA_FP4_E2M1_MX;
    timed_launch(HSA_K_INDEXER_GEMM,
                 s16 ? (f8k   ? idx_gemm_kernel<true, false, true>
                        : f4k ? idx_gemm_kernel<false, true, true> : idx_gemm_kernel<false, false, true>)
                     : (f8k   ? idx_gemm_kernel<true, false, false>
                        : f4k ? idx_gemm_kernel<false, true, false>
                              : idx_gemm_kernel<false, false, false>),
                 dim3(bsplit, (nq + 15) / 16), dim3(256), 0,
                 s, Qd, q0, nq, (const u16*)qI, w, kc, m, n_win, ws, fault);
    KernelTimer kt(HSA_K_INDEXER_SEL, s);
    const dim3 hgrid(nv_hi > kHistSpan ? (unsigned)((nv_hi + kHistSpan - 1) / kHistSpan) : 1u, nq);
    // rows the one-kernel selection takes build their histograms themselves;
    // longer rows merge the lists of the histogram kernel
    const bool self_hist = R <= kFusedMaxBlocksPrefill;
    if (s16) {
      if (!self_hist) idx_hist_kernel<true><<<hgrid, 256, 0, s>>>(Qd, q0, kc, m, n_win, k, ws, fault);
      launch_topk<true>(256, nq, k, ws, idx, score, q0, s, self_hist);
    } else {
      if (!self_hist) idx_hist_kernel<false><<<hgrid, 256, 0, s>>>(Qd, q0, kc, m, n_win, k, ws, fault);
      launch_topk<false>(256, nq, k, ws, idx, score, q0, s, self_hist);
    }
  }
  return hipGetLastError();
}

}  // namespace hsa
