// Gather + online-softmax attention for CSA and HCA over one shared KV head.
//
// Each query token attends, with one softmax, to its window rows (raw bf16
// tokens s(t)..t) followed by compressed entries: the top-k selection (CSA)
// or every visible block (HCA).  All query heads share the same rows (MQA), so
// the heads form the N dimension of MFMA 16x16x32 bf16 tiles:
//   S^T[e][h]  = K[e][:] . Q[h][:]     A = K rows from LDS, B = Q in registers (bf16)
//   O^T[c][h] += V^T[c][e] * P^T[e][h] A = V^T from LDS,  B = P in registers (fp16)
// With heads as columns, a lane owns one head in both products, so the
// running max, the row sums and the rescaling of O stay in-lane (two lane
// swaps finish each reduction), and the probabilities feed the second product
// straight from the registers of the first: the k index of the second
// product visits entries in the order the first product's result rows sit in
// a lane, and V^T is read from LDS in that same order.
//
// Rows are gathered 64 entries at a time into LDS (K row-major, V transposed).
// K stays bf16 (fp8 e4m3 codes widen to bf16 exactly; the page scale multiplies
// the logits).  The second product runs in fp16: bf16 V values (and fp8 codes
// times their page scale) become fp16 -- exact for bf16 magnitudes in
// [2^-14, 65504] -- and the probabilities keep 10 fraction bits instead of 7,
// which keeps the output error well inside what the bf16 output store adds.
// Long decode rows are split over workgroups and merged through (max, sum,
// normalized partial O) in the workspace: a split stores o = O / sum in fp16
// (|o| <= max |v|, which the fp16 V staging already bounds), halving the
// partial traffic; a decode query whose entries fit one split divides exactly
// as the merge does, so its bits do not depend on the batch around it.
#include <type_traits>

#include "update.h"

namespace hsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  Queries Q;
  const u16* q;
  int H;
  Tokens wk, wv;
  int n_win;
  Paged kc, vc;
  int m;
  const int32_t* idx;
  int k;                 // > 0: CSA selection of width k; 0: HCA (all visible)
  float scale_log2;      // logit scale times log2(e)
  void* O;
  int o_f32;             // 1: fp32 output, 0: bf16
  float* lse;
  u16* part_o;           // fp16 [n][splits][H][128]: o = O / sum of the split
  float* part_ml;        // [n][splits][H][2]: (max, sum)
  int n_splits, cps, n_hg, n_q;
  int xcd;               // 1: keep consecutive queries on one XCD (prefill)
  int pt_lds;            // 1: CSA decode reads the request's page tables into LDS
  int* fault;
  // decode with the cache upkeep after the attention: the query's own token
  // (the newest window row) is read from row qi of knew / vnew instead of the
  // ring, where it is not yet written; its F8 row id is -2 - (ring_rows + qi)
  const u16* knew;
  const u16* vnew;
  int64_t ring_rows;     // n_req * capacity of the rings
};

constexpr int kMaxCps = 32;            // chunks of 64 entries per workgroup
constexpr int kZeroRow = -1;          // reads as zeros (neither a pool nor a window row)

// Row id of entry ge of a query: >= 0 is a row of the paged pool (page*64 + slot);
// <= -2 encodes window row w as -2 - w; kZeroRow (-1) reads as zeros.
struct Prefetch;
__device__ __forceinline__ int64_t entry_block(const AttnArgs& a, const Prefetch& pf, int qi, int j);
__device__ __forceinline__ int entry_page(const AttnArgs& a, const Paged& c, const Prefetch& pf,
                                          int which, int r, int64_t b);

// Ring slot of window row ge: the window start's slot w0 (= s0 mod capacity,
// computed once per workgroup) plus ge, wrapped once (ge < n_win <= capacity)
__device__ __forceinline__ int64_t ring_slot(int64_t w0, int ge, int64_t cap) {
  const int64_t sl = w0 + ge;
  return sl >= cap ? sl - cap : sl;
}

template <bool NR>
__device__ __forceinline__ void resolve(const AttnArgs& a, const Prefetch& pf, int qi, int r,
                                        int64_t w0k, int64_t w0v, int n_w, int E, int64_t nv,
                                        int ge, int* rk, int* rv) {
  if (ge < n_w) {
    if (NR && ge == n_w - 1) {   // the query's own token, from knew / vnew
      *rk = *rv = -2 - (int)(a.ring_rows + qi);
      return;
    }
    *rk = -2 - (int)((int64_t)r * a.wk.capacity + ring_slot(w0k, ge, a.wk.capacity));
    *rv = -2 - (int)((int64_t)r * a.wv.capacity + ring_slot(w0v, ge, a.wv.capacity));
    return;
  }
  *rk = *rv = kZeroRow;
  if (ge >= E) return;
  const int64_t b = entry_block(a, pf, qi, ge - n_w);
  if (b < 0 || b >= nv) {
    atomicOr(a.fault, HSA_FAULT_INDEX);
    return;
  }
  const int pk = entry_page(a, a.kc, pf, 0, r, b), pv = entry_page(a, a.vc, pf, 1, r, b);
  if (pk >= 0) *rk = pk * kPage + (int)(b & 63);
  if (pv >= 0) *rv = pv * kPage + (int)(b & 63);
}

// Decode: what the rows of a split's entries depend on, loaded before the
// query's position is known, over the span of entries the split can cover for
// any window length 1..n_win: its top-k ids (CSA) or the page ids of its blocks
// (HCA).  Lives in dynamic LDS.
struct Prefetch {
  const int* p;       // LDS, or nullptr (prefill: look up directly)
  int lo;             // CSA: first idx position held; HCA: first page held
  int n;              // entries held (CSA: idx positions; HCA: pages, K at p[i], V at p[64 + i])
  const int* pt;      // CSA decode: the request's page table rows in LDS (K, then V), or nullptr
  int pt_k;           // K page-table entries held (V's follow them)
};
constexpr int kPrePages = 64;   // HCA: page ids held per cache
constexpr int kPtLdsMax = 4096; // CSA decode: page-table entries per cache read into LDS

// block id of compressed entry j of query qi (CSA: its top-k id), or -1
__device__ __forceinline__ int64_t entry_block(const AttnArgs& a, const Prefetch& pf, int qi,
                                               int j) {
  if (a.k <= 0) return j;
  if (pf.p && j >= pf.lo && j < pf.lo + pf.n) return pf.p[j - pf.lo];
  return a.idx[(int64_t)qi * a.k + j];
}

// physical page of block b of request r in cache c (which = 0: K, 1: V), or -1
__device__ __forceinline__ int entry_page(const AttnArgs& a, const Paged& c, const Prefetch& pf,
                                          int which, int r, int64_t b) {
  if (pf.p && a.k <= 0) {
    const int i = (int)(b >> 6) - pf.lo;
    if (i >= 0 && i < pf.n) {
      const int p = pf.p[which * kPrePages + i];
      if ((unsigned)p < (unsigned)c.n_pages) return p;
      atomicOr(a.fault, HSA_FAULT_PAGE);
      return -1;
    }
  }
  if (pf.pt) {   // (b < n_vis <= pages_per_req * 64: the entry is held)
    const int p = pf.pt[(which ? pf.pt_k : 0) + (int)(b >> 6)];
    if ((unsigned)p < (unsigned)c.n_pages) return p;
    atomicOr(a.fault, HSA_FAULT_PAGE);
    return -1;
  }
  return c.page_of(r, b, a.fault);
}

// 256 bytes of zeros: the row read for entries past the end of a query's list
__device__ __align__(16) uint4 g_zero_row[16];

// bf16 caches: the address of entry ge's K and V rows (window row, pool row, or
// the zero row), so that a chunk's gathers are one load per 16-byte piece.
template <bool NR>
__device__ __forceinline__ void resolve_ptr(const AttnArgs& a, const Prefetch& pf, int qi, int r,
                                            int64_t w0k, int64_t w0v, int n_w, int E, int64_t nv,
                                            int ge, const uint8_t** pk, const uint8_t** pv) {
  const uint8_t* zero = (const uint8_t*)g_zero_row;
  if (ge < n_w) {
    if (NR && ge == n_w - 1) {   // the query's own token, from knew / vnew
      *pk = (const uint8_t*)(a.knew + (int64_t)qi * kD);
      *pv = (const uint8_t*)(a.vnew + (int64_t)qi * kD);
      return;
    }
    *pk = a.wk.data + ((int64_t)r * a.wk.capacity + ring_slot(w0k, ge, a.wk.capacity)) * (kD * 2);
    *pv = a.wv.data + ((int64_t)r * a.wv.capacity + ring_slot(w0v, ge, a.wv.capacity)) * (kD * 2);
    return;
  }
  *pk = *pv = zero;
  if (ge >= E) return;
  const int64_t b = entry_block(a, pf, qi, ge - n_w);
  if (b < 0 || b >= nv) {
    atomicOr(a.fault, HSA_FAULT_INDEX);
    return;
  }
  const int pgk = entry_page(a, a.kc, pf, 0, r, b), pgv = entry_page(a, a.vc, pf, 1, r, b);
  if (pgk >= 0) *pk = a.kc.data + ((int64_t)pgk * kPage + (b & 63)) * (kD * 2);
  if (pgv >= 0) *pv = a.vc.data + ((int64_t)pgv * kPage + (b & 63)) * (kD * 2);
}

// Raw 16 bytes (bf16) or 8 bytes (fp8 codes, in .x/.y) of column group cg of a
// row.  Branch-free: both the window row and the pool row are loaded from
// always-valid addresses (row 0 stands in for the one not used) and the right
// one is selected afterwards, so the loads of a chunk stay in flight together
// instead of waiting at divergent branch joins (measured: a variant that
// issues one load on chunks that lie wholly in the window or the pool, behind
// a chunk-uniform branch, is 10-30% slower).
template <bool F8, bool NR>
__device__ __forceinline__ uint4 load_piece(const Paged& c, const Tokens& tk, int row, int cg,
                                            const u16* knew, int64_t ring_rows) {
  const bool pool = row >= 0, win = row <= -2;
  const int64_t pr = pool ? row : 0;
  const int64_t w = win ? (int64_t)(-2 - row) : 0;
  const bool nw = NR && w >= ring_rows;       // the query's own token
  const u16* wb = nw ? knew : (const u16*)tk.data;
  const int64_t wr = nw ? w - ring_rows : w;
  const uint4 wv = *(const uint4*)(wb + wr * kD + cg * 8);
  uint4 pv;
  if (F8) {
    const uint2 v = *(const uint2*)(c.data + pr * kD + cg * 8);
    pv = make_uint4(v.x, v.y, 0, 0);
  } else {
    pv = *(const uint4*)(c.data + (pr * kD + cg * 8) * 2);
  }
  const uint4 z = make_uint4(0, 0, 0, 0);
  return pool ? pv : (win ? wv : z);
}

// Column group cg of a K row of an HSA_FP8_BF16_ROPE cache (the window rows
// are bf16): groups 0-7 are fp8 codes (8 bytes, in .x/.y), groups 8-15 the bf16
// RoPE channels.  One 16-byte load per piece, branch-free like load_piece: a
// code group reads the 16 bytes that hold it and its neighbour and keeps its
// half.
template <bool NR>
__device__ __forceinline__ uint4 load_piece_kmix(const Paged& c, const Tokens& tk, int row,
                                                 int cg, const u16* knew, int64_t ring_rows) {
  const bool pool = row >= 0, win = row <= -2;
  const int64_t pr = pool ? row : 0;
  const int64_t w = win ? (int64_t)(-2 - row) : 0;
  const bool nw = NR && w >= ring_rows;       // the query's own token
  const u16* wb = nw ? knew : (const u16*)tk.data;
  const int64_t wr = nw ? w - ring_rows : w;
  const uint4 wv = *(const uint4*)(wb + wr * kD + cg * 8);
  const uint8_t* base = c.data + pr * (kD / 2 * 3);
  const bool code = cg < 8;
  const uint4 v = *(const uint4*)(base + (code ? (cg >> 1) * 16 : kD / 2 + (cg - 8) * 16));
  const uint4 cv = (cg & 1) ? make_uint4(v.z, v.w, 0, 0) : make_uint4(v.x, v.y, 0, 0);
  const uint4 pv = code ? cv : v;
  const uint4 z = make_uint4(0, 0, 0, 0);
  return pool ? pv : (win ? wv : z);
}

template <bool F8>
__device__ __forceinline__ float row_scale(const Paged& c, int row) {
  if (!F8) return 1.f;
  const float sc = c.scale[(row >= 0 ? row : 0) >> 6];
  return row >= 0 ? sc : 1.f;
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __fp16 f16x2v __attribute__((ext_vector_type(2)));

// 8 e4m3fn codes (two 32-bit words) -> 8 floats, by the hardware converter
// (exact: every e4m3 value is an fp32 value).
__device__ __forceinline__ void fp8x8_to_f32(uint32_t lo, uint32_t hi, float f[8]) {
  f32x2v a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  f32x2v b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  f32x2v c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  f32x2v d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y; f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// 16 bytes from a global-memory address held as an integer (a global, not a
// flat, load: flat loads also count against the LDS wait counter, which would
// make every LDS wait in the chunk loop wait for the next chunk's gathers too)
__device__ __forceinline__ uint4 gload16(uintptr_t addr) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 2^x with the hardware instruction alone (results below 2^-126 flush to zero,
// far below what the fp16 probabilities can hold)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// two floats -> packed fp16, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{x, y}), h2));
}

// K piece -> 8 bf16 (fp8 codes widen exactly: keep the upper half of the float)
__device__ __forceinline__ uint4 k_piece_bf16(uint4 raw, bool fp8) {
  if (!fp8) return raw;
  float f[8];
  fp8x8_to_f32(raw.x, raw.y, f);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xFFFF0000u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// V piece -> 8 fp16 values (fp8 codes times the page scale, rounded once to
// nearest; bf16 values are exact in the fp16 range)
__device__ __forceinline__ uint4 v_piece_f16(uint4 raw, bool fp8, float scale) {
  float f[8];
  if (fp8) {
    fp8x8_to_f32(raw.x, raw.y, f);
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = (uint32_t)__builtin_bit_cast(u16, (_Float16)(f[2 * i] * scale)) |
             ((uint32_t)__builtin_bit_cast(u16, (_Float16)(f[2 * i + 1] * scale)) << 16);
    return make_uint4(h[0], h[1], h[2], h[3]);
  }
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return make_uint4(pack_f16(f[0], f[1]), pack_f16(f[2], f[3]), pack_f16(f[4], f[5]),
                    pack_f16(f[6], f[7]));
}

// Raise HSA_FAULT_RANGE when an output accumulator is not finite: V values are
// staged in fp16 for the P V product, so a |v| above 65504 (or a non-finite
// input) turns the affected outputs into inf / NaN; the fault word reports it.
template <int N>
__device__ __forceinline__ void check_finite(const f32x4 (&acc)[N], int* fault) {
  bool bad = false;
#pragma unroll
  for (int i = 0; i < N; ++i)
    bad |= !(__builtin_isfinite(acc[i][0]) && __builtin_isfinite(acc[i][1]) &&
             __builtin_isfinite(acc[i][2]) && __builtin_isfinite(acc[i][3]));
  if (bad) atomicOr(fault, HSA_FAULT_RANGE);
}

// KMIX (with F8): the K cache is HSA_FP8_BF16_ROPE, the V cache fp8
// NR: decode with the upkeep after the attention (the query's own token read
// from knew / vnew)
template <int NW, bool F8, bool SH, bool KMIX, bool NR = false>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int PPT = 1024 / NT;          // K (and V) pieces per thread per chunk
  unsigned bid = blockIdx.x;
  if (a.xcd) {
    // blocks are handed to the 8 XCDs round-robin; give each XCD a contiguous
    // range of queries so window rows and compressed entries stay in its L2
    unsigned per = gridDim.x / 8;
    bid = (bid % 8) * per + bid / 8;
  }
  const int split = bid % a.n_splits;
  const int rest = bid / a.n_splits;
  const int hg = rest % a.n_hg;
  const int qi = rest / a.n_hg;
  if (qi >= a.n_q) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  // the query rows depend on nothing else: requested first
  const int head = hg * 16 * NW + wave * 16 + col;
  bf16x8 qb[4];
  {
    const bf16x8* qp = (const bf16x8*)(a.q + ((int64_t)qi * a.H + head) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = qp[4 * ks + g];
  }
  // the position, the request's entry counts and -- decode -- what the rows
  // depend on (top-k ids, or page ids) are requested together, before any of
  // them is used: one memory round trip.  The ids are loaded first, into
  // registers, and the position and counts last: those are uniform values the
  // compiler waits for as soon as they are loaded, and loads complete in
  // order, so that one wait covers every load.
  const bool listed = a.Q.pos != nullptr;
  const int r = a.Q.req_of(qi, a.fault);
  // dynamic LDS: the row ids of the split's entries (K, then V), then -- decode
  // launches -- the prefetched top-k or page ids
  // (fp8: 32-bit row ids, pool rows holding fp8 codes and window rows bf16;
  // bf16: row addresses)
  typedef typename std::conditional<F8, int, const uint8_t*>::type RowT;
  extern __shared__ __align__(16) int dyn_lds[];
  RowT* rowk = (RowT*)dyn_lds;
  RowT* rowv = rowk + a.cps * 64;
  int* spre = (int*)(rowv + a.cps * 64);
  const int e_nom = split * a.cps * 64, n_nom = a.cps * 64;
  // CSA: top-k positions [pre_lo, pre_lo + n_pre); HCA (one query per request,
  // in request order): pages [pre_lo, pre_lo + n_pre) of both caches
  const int pre_mode = a.xcd ? 0 : (a.k > 0 ? 1 : (!a.Q.req ? 2 : 0));
  int pre_lo = 0, n_pre = 0;
  if (pre_mode == 1) {
    pre_lo = e_nom - a.n_win > 0 ? e_nom - a.n_win : 0;
    const int hi = e_nom + n_nom < a.k ? e_nom + n_nom : a.k;
    n_pre = hi > pre_lo ? hi - pre_lo : 0;
  } else if (pre_mode == 2) {
    pre_lo = e_nom - a.n_win > 0 ? (e_nom - a.n_win) >> 6 : 0;
    const int n = ((e_nom + n_nom - 1) >> 6) + 1 - pre_lo;
    n_pre = n < kPrePages ? n : kPrePages;
  }
  int id_a = -1, id_b = -1;   // this thread's first ids (K and V pages, or one top-k id)
  if (tid < n_pre) {
    if (pre_mode == 1) {
      id_a = a.idx[(int64_t)qi * a.k + pre_lo + tid];
    } else {
      // clamped in-bounds reads (pages_per_req >= 1), masked below
      const int lp = pre_lo + tid;
      const int lk = lp < a.kc.pages_per_req ? lp : a.kc.pages_per_req - 1;
      const int lv = lp < a.vc.pages_per_req ? lp : a.vc.pages_per_req - 1;
      id_a = a.kc.page_table[(int64_t)r * a.kc.pages_per_req + lk];
      id_b = a.vc.page_table[(int64_t)r * a.vc.pages_per_req + lv];
    }
  }
  // CSA decode (a.pt_lds: the request is the query's index, no load): the
  // request's page-table rows of both caches are read with the ids, so the
  // rows of the selected blocks resolve from LDS instead of through a page
  // table read that waits for the ids (one round trip fewer).  Whole rounds
  // past both rows are skipped (uniform); the rest read clamped addresses.
  constexpr int PTT = NW >= 4 ? kPtLdsMax / NT : 1;
  const bool pt_lds = NW >= 4 && pre_mode == 1 && a.pt_lds;
  const int ppk = a.kc.pages_per_req, ppv = a.vc.pages_per_req;
  const int pp_max = ppk > ppv ? ppk : ppv;
  int ptk_r[PTT], ptv_r[PTT];
  if (pt_lds) {
#pragma unroll
    for (int i = 0; i < PTT; ++i) {
      if (i * NT < pp_max) {
        const int j = tid + NT * i;
        ptk_r[i] = a.kc.page_table[(int64_t)r * ppk + (j < ppk ? j : ppk - 1)];
        ptv_r[i] = a.vc.page_table[(int64_t)r * ppv + (j < ppv ? j : ppv - 1)];
      }
    }
  }
  const int64_t ne_k = a.kc.n_entries[r], ne_v = a.vc.n_entries[r];
  const int64_t p_raw = listed ? a.Q.pos[qi] : a.Q.span_pos0 + qi;
  Prefetch pf{nullptr, 0, 0, nullptr, 0};
  if (pre_mode != 0) {
    if (tid < n_pre) {
      if (pre_mode == 1) {
        spre[tid] = id_a;
      } else {
        const int lp = pre_lo + tid;
        spre[tid] = lp < a.kc.pages_per_req ? id_a : -1;
        spre[kPrePages + tid] = lp < a.vc.pages_per_req ? id_b : -1;
      }
    }
    if (pre_mode == 1)   // top-k ranges longer than the workgroup
      for (int i = tid + NT; i < n_pre; i += NT) spre[i] = a.idx[(int64_t)qi * a.k + pre_lo + i];
    pf = Prefetch{spre, pre_lo, n_pre, nullptr, 0};
    if (pt_lds) {
      int* spt = spre + a.cps * 64 + a.n_win + 2 * kPrePages;
#pragma unroll
      for (int i = 0; i < PTT; ++i) {
        if (i * NT < pp_max) {
          const int j = tid + NT * i;
          if (j < ppk) spt[j] = ptk_r[i];
          if (j < ppv) spt[ppk + j] = ptv_r[i];
        }
      }
      pf.pt = spt;
      pf.pt_k = ppk;
    }
  }
  if (!a.xcd) __syncthreads();
  int64_t t = p_raw;
  if (listed && (t > a.Q.max_pos || t < 0)) {
    atomicOr(a.fault, HSA_FAULT_POS);
    t = t < 0 ? 0 : a.Q.max_pos;
  }
  const int64_t s0 = window_start(t, a.n_win);
  const int n_w = (int)(t - s0 + 1);
  int64_t nv = n_visible(t, a.m, a.n_win);
  {
    const int64_t ne = ne_k < ne_v ? ne_k : ne_v;
    if (nv > ne) {
      if (split == 0 && hg == 0 && tid == 0) atomicOr(a.fault, HSA_FAULT_ENTRIES);
      nv = ne < 0 ? 0 : ne;
    }
  }
  const int n_c = a.k > 0 ? (int)(nv < a.k ? nv : a.k) : (int)nv;
  // E is the same in every lane; saying so keeps the chunk loop's conditions
  // (last-chunk masking, loop bounds) scalar branches instead of selects
  const int E = __builtin_amdgcn_readfirstlane(n_w + n_c);
  const int n_chunks = (E + 63) / 64;
  const int c_lo = split * a.cps;
  const int c_hi = c_lo + a.cps < n_chunks ? c_lo + a.cps : n_chunks;

  // K tile (row-major bf16) and V^T tile (fp16 bits).  SH: one buffer for both,
  // V^T staged once every wave has read the K tile (half the LDS, so more
  // workgroups fit on a CU, for two more barriers per chunk).  V^T row pitch:
  // SH (the prefill) 34 dwords, which spreads the 16 rows one P V operand
  // read touches over distinct bank pairs (36 put rows r and r + 8 on the
  // same banks: 4% of the prefill attention time); decode keeps 36, measured
  // as fast or faster there
  constexpr int kVtP = SH ? 68 : 72;
  constexpr int kKsH = 64 * 136, kVtH = 128 * kVtP;
  __shared__ __align__(16) u16 kv_lds[SH ? (kVtH > kKsH ? kVtH : kKsH) : kKsH + kVtH];
  u16(*Ks)[136] = (u16(*)[136])kv_lds;
  u16(*Vt)[kVtP] = (u16(*)[kVtP])(kv_lds + (SH ? 0 : kKsH));
  __shared__ __align__(16) float ksc[64];

  // ---- resolve the rows of every entry of this split once
  const int e_base = c_lo * 64;
  const int n_ent = (c_hi > c_lo) ? (c_hi - c_lo) * 64 : 0;
  // the window start's ring slots: one division per workgroup (s0 is uniform)
  const int64_t w0k = mod_nn(s0, a.wk.capacity), w0v = mod_nn(s0, a.wv.capacity);
  for (int j = tid; j < n_ent; j += NT) {
    if constexpr (F8)
      resolve<NR>(a, pf, qi, r, w0k, w0v, n_w, E, nv, e_base + j, &rowk[j], &rowv[j]);
    else
      resolve_ptr<NR>(a, pf, qi, r, w0k, w0v, n_w, E, nv, e_base + j, &rowk[j], &rowv[j]);
  }

  __syncthreads();

  // ---- register buffers of a chunk's rows.  K pieces: p = tid + NT*i is
  // (entry p/16, column group p%16).  V pieces: this thread's entry pair
  // (2*(tid%32), +1) in column groups tid/32 + (NT/32)*j, so that two entries
  // share one 32-bit word of the transposed tile.  Decode keeps DEPTH = 2
  // chunks of gathers in flight (chunk c + 2 loads while chunk c computes);
  // prefill (SH) one, its registers going to occupancy instead.  The buffer
  // index is always a compile-time constant (the chunk loop is unrolled by
  // DEPTH), so the arrays stay in registers.
  constexpr int DEPTH = (SH || NW < 4) ? 1 : 2;
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  uint4 kraw[DEPTH][PPT], vraw[DEPTH][PPT];
  int krow[DEPTH][PPT], vrow[DEPTH][PPT];
  float kscl[DEPTH][PPT], vscl[DEPTH][PPT];
  const int vpair = tid & 31;
  auto issue_k = [&](int c, auto bi) {
    constexpr int b = decltype(bi)::value;
    const int lo = (c - c_lo) * 64;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      const int ek = p >> 4, cgk = p & 15;
      if constexpr (F8) {
        krow[b][i] = rowk[lo + ek];
        kraw[b][i] = KMIX ? load_piece_kmix<NR>(a.kc, a.wk, krow[b][i], cgk, a.knew, a.ring_rows)
                          : load_piece<F8, NR>(a.kc, a.wk, krow[b][i], cgk, a.knew, a.ring_rows);
        kscl[b][i] = row_scale<F8>(a.kc, krow[b][i]);
      } else {
        krow[b][i] = 0;
        kscl[b][i] = 1.f;
        kraw[b][i] = gload16((uintptr_t)rowk[lo + ek] + cgk * 16);
      }
    }
  };
  auto issue_v = [&](int c, auto bi) {
    constexpr int b = decltype(bi)::value;
    const int lo = (c - c_lo) * 64;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int ev = 2 * vpair + (i & 1), cgv = (tid >> 5) + (NT / 32) * (i >> 1);
      if constexpr (F8) {
        vrow[b][i] = rowv[lo + ev];
        vraw[b][i] = load_piece<F8, NR>(a.vc, a.wv, vrow[b][i], cgv, a.vnew, a.ring_rows);
        vscl[b][i] = row_scale<F8>(a.vc, vrow[b][i]);
      } else {
        vrow[b][i] = 0;
        vscl[b][i] = 1.f;
        vraw[b][i] = gload16((uintptr_t)rowv[lo + ev] + cgv * 16);
      }
    }
  };

  float m_i = -1e30f;
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 osum = {0.f, 0.f, 0.f, 0.f};       // row sums of P (every row of the tile)
  f16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;

  // V (transposed fp16) of the chunk in buffer b -> Vt
  auto stage_v = [&](auto bi) {
    constexpr int b = decltype(bi)::value;
#pragma unroll
    for (int j = 0; j < PPT / 2; ++j) {
      const int cgv = (tid >> 5) + (NT / 32) * j;
      const uint4 v0 = v_piece_f16(vraw[b][2 * j], F8 && vrow[b][2 * j] >= 0, vscl[b][2 * j]);
      const uint4 v1 =
          v_piece_f16(vraw[b][2 * j + 1], F8 && vrow[b][2 * j + 1] >= 0, vscl[b][2 * j + 1]);
      const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
      uint32_t* vt = (uint32_t*)&Vt[cgv * 8][0] + vpair;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        vt[(2 * q2) * (kVtP / 2)] = (a0[q2] & 0xFFFFu) | (a1[q2] << 16);
        vt[(2 * q2 + 1) * (kVtP / 2)] = (a0[q2] >> 16) | (a1[q2] & 0xFFFF0000u);
      }
    }
  };

  // one chunk from buffer b; then buffer b receives chunk c + DEPTH
  auto body = [&](int c, auto bi) {
    constexpr int b = decltype(bi)::value;
    const int e0 = c * 64;
    // ---- stage K (row-major bf16), and V unless it waits for the K tile's reads
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      const int ek = p >> 4, cgk = p & 15;
      *(uint4*)&Ks[ek][cgk * 8] =
          k_piece_bf16(kraw[b][i], F8 && krow[b][i] >= 0 && (!KMIX || cgk < 8));
      // page scale of each key row (bf16 rows need none); fp8 K: times the
      // logit scale, the product the softmax takes (the same fp32 value)
      if constexpr (F8)
        if (cgk == 0) ksc[ek] = KMIX ? kscl[b][i] : a.scale_log2 * kscl[b][i];
    }
    if constexpr (!SH) stage_v(bi);
    __syncthreads();
    // chunk c + DEPTH loads while this one computes
    if (c + DEPTH < c_hi) {
      issue_k(c + DEPTH, bi);
      if constexpr (!SH) issue_v(c + DEPTH, bi);
    }
    // ---- S^T = K Q^T for 64 entries x 16 heads (this wave's heads).  KMIX:
    // the code channels (k-steps 0, 1) and the bf16 RoPE channels (2, 3)
    // accumulate apart, as only the codes take the page scale.
    // every K operand of the chunk is read from LDS before the first MFMA
    // (one LDS round trip instead of one per operand), and the four entry
    // tiles' accumulations interleave
    f32x4 sacc[4], shi[KMIX ? 4 : 1];
    bf16x8 kf[4][4];
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[et][ks] = *(const bf16x8*)&Ks[et * 16 + col][ks * 32 + 8 * g];
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      sacc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KMIX) shi[et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        if (KMIX && ks >= 2)
          shi[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[et][ks], qb[ks], shi[et], 0, 0, 0);
        else
          sacc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[et][ks], qb[ks], sacc[et], 0, 0, 0);
      }
    // ---- online softmax (lane = head `col`; rows 4g+i of each entry tile).
    // log2-domain logit = acc * c, c = scale*log2(e) (times the page scale of
    // fp8 keys).  With one positive c the running max is taken on the raw
    // accumulators; entries past the end exist only in the last chunk.
    if (F8) {
      // the key rows' page scales, four per 16-byte read
      f32x4 kscv[4];
#pragma unroll
      for (int et = 0; et < 4; ++et) kscv[et] = *(const f32x4*)&ksc[et * 16 + 4 * g];
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (KMIX)
            sacc[et][i] = (sacc[et][i] * kscv[et][i] + shi[et][i]) * a.scale_log2;
          else
            sacc[et][i] *= kscv[et][i];
        }
    }
    if (__builtin_expect(e0 + 64 > E, 0)) {   // the last chunk only (E is uniform)
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e0 + et * 16 + 4 * g + i >= E) sacc[et][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[et][i]);
    if (!F8) mx *= a.scale_log2;
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
    m_i = m_new;
    const float cst = F8 ? 1.f : a.scale_log2;
    // the running max rarely grows once a row is under way: skip the rescale
    // when no lane of the wave needs it (alpha is exactly 1 then)
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
      osum *= alpha;
    }

    if constexpr (SH) {
      __syncthreads();   // every wave has read the K tile
      stage_v(bi);
      __syncthreads();
      if (c + DEPTH < c_hi) issue_v(c + DEPTH, bi);
    }
    // ---- O^T += V^T P^T, two k-steps of 32 entries.  P is rounded to fp16
    // once; an extra tile of ones in place of V^T rows accumulates the row
    // sums of exactly those rounded weights.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        pw[i / 2] = pack_f16(ex2(__builtin_fmaf(sacc[2 * j][i], cst, -m_new)),
                             ex2(__builtin_fmaf(sacc[2 * j][i + 1], cst, -m_new)));
        pw[2 + i / 2] = pack_f16(ex2(__builtin_fmaf(sacc[2 * j + 1][i], cst, -m_new)),
                                 ex2(__builtin_fmaf(sacc[2 * j + 1][i + 1], cst, -m_new)));
      }
      const f16x8 pb = __builtin_bit_cast(f16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      // the step's V^T operands, all read before the MFMAs use them
      f16x8 vf[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u16* vr = &Vt[16 * dt + col][0];
        uint2 lo = *(const uint2*)(vr + 32 * j + 4 * g);
        uint2 hi = *(const uint2*)(vr + 32 * j + 16 + 4 * g);
        vf[dt] = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], pb, oacc[dt], 0, 0, 0);
      // schedule: the step's LDS reads (8 pairs) ahead of its MFMAs, so their
      // latencies overlap instead of one wait per operand
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // MFMA
      osum = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb, osum, 0, 0, 0);
    }
    __syncthreads();
  };

  if (c_lo < c_hi) {
    issue_k(c_lo, B0{});
    issue_v(c_lo, B0{});
  }
  if constexpr (DEPTH == 2) {
    if (c_lo + 1 < c_hi) {
      issue_k(c_lo + 1, B1{});
      issue_v(c_lo + 1, B1{});
    }
    for (int c = c_lo; c < c_hi; c += 2) {
      body(c, B0{});
      if (c + 1 < c_hi) body(c + 1, B1{});
    }
  } else {
    for (int c = c_lo; c < c_hi; ++c) body(c, B0{});
  }
  const float l_i = osum[0];
  check_finite(oacc, a.fault);

  // ---- epilogue: lane holds O^T[16dt + 4g + i][head]
  // the split's normalized output, rounded to fp16 (0 for an empty split)
  const bool nz = l_i > 0.f;
  const bool listed_q = a.Q.pos != nullptr;
  if (a.n_splits == 1) {
    // decode: (l * fp16(O / l)) / l, the merge's arithmetic for a query with one
    // non-empty split, so a query's bits do not depend on its batch; prefill
    // (spans, never split): O / l
    const int64_t o0 = ((int64_t)qi * a.H + head) * kD;
    float ov[8][4];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = nz ? oacc[dt][i] / l_i : 0.f;
        const float o16 = (float)(_Float16)o;
        ov[dt][i] = !listed_q ? o : (nz ? (l_i * o16) / l_i : 0.f);
      }
    if (a.o_f32) {
      float* orow = (float*)a.O + o0;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(f32x4*)(orow + 16 * dt + 4 * g) = f32x4{ov[dt][0], ov[dt][1], ov[dt][2], ov[dt][3]};
    } else {
      u16* orow = (u16*)a.O + o0;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(u16, (__bf16)ov[dt][i]);
        *(uint2*)(orow + 16 * dt + 4 * g) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
    if (g == 0 && a.lse) a.lse[(int64_t)qi * a.H + head] = (m_i + log2f(l_i)) * kLn2;
  } else {
    const int64_t slot = ((int64_t)qi * a.n_splits + split) * a.H + head;
    u16* po = a.part_o + slot * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *(uint2*)(po + 16 * dt + 4 * g) =
          make_uint2(pack_f16(nz ? oacc[dt][0] / l_i : 0.f, nz ? oacc[dt][1] / l_i : 0.f),
                     pack_f16(nz ? oacc[dt][2] / l_i : 0.f, nz ? oacc[dt][3] / l_i : 0.f));
    if (g == 0) {
      a.part_ml[slot * 2 + 0] = m_i;
      a.part_ml[slot * 2 + 1] = l_i;
    }
  }
}

// Merge split partials: O = sum_s w_s o_s / sum_s w_s, w_s = 2^(m_s - M) l_s,
// with o_s the split's normalized fp16 output.  One wave per (query, head):
// lane j owns output dims 2j, 2j+1 (one 4-byte load of two fp16 values per
// split) and split s's (m, l) sits in lane s mod 64, so every reduction stays
// inside the wave and a split's place in it does not depend on how many
// splits the launch has.  The first kMergePF partial rows are requested before
// the (m, l) pairs are reduced.  Every thread of the workgroup calls it (one
// workgroup barrier); `on` false: a wave with no (query, head).
constexpr int kMergeMaxSplits = 1024;
constexpr int kMergePF = 64;          // partial rows a lane requests up front (HCA: 44 splits at 1M)
__device__ __forceinline__ void merge_one(int qh, bool on, int H, int n_splits,
                                          const u16* __restrict__ part_o,
                                          const float* __restrict__ part_ml, void* __restrict__ O,
                                          int o_f32, float* __restrict__ lse, int* fault,
                                          float* wgt, float* wls) {
  const int lane = threadIdx.x & 63;
  const int q = on ? qh / H : 0, h = on ? qh % H : 0;
  const int ns = !on ? 0 : (n_splits < kMergeMaxSplits ? n_splits : kMergeMaxSplits);
  const uint32_t* po = (const uint32_t*)(part_o + ((int64_t)q * n_splits * H + h) * kD) + lane;
  const int64_t stride = (int64_t)H * kD / 2;    // 32-bit words between splits
  uint32_t v[kMergePF];
#pragma unroll
  for (int j = 0; j < kMergePF; ++j) v[j] = j < ns ? po[j * stride] : 0u;
  // each split's (max, sum) pair is read once: the max to wgt[], the sum to
  // wls[] (the lane that reads them is the lane that uses them)
  float mloc = -INFINITY;
  for (int s = lane; s < ns; s += 64) {
    const float2 ml = *(const float2*)&part_ml[(((int64_t)q * n_splits + s) * H + h) * 2];
    wgt[s] = ml.x;
    wls[s] = ml.y;
    mloc = fmaxf(mloc, ml.x);
  }
  const float M = wave_max_f32(mloc);
  float lloc = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float wl = exp2f(wgt[s] - M) * wls[s];
    wgt[s] = wl;
    lloc += wl;
  }
  const float L = wave_sum_f32(lloc);
  __syncthreads();   // wgt[] written by other lanes
  if (!on) return;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < kMergePF; ++j)
    if (j < ns) {
      const h2 x = __builtin_bit_cast(h2, v[j]);
      a0 += wgt[j] * (float)x.x;
      a1 += wgt[j] * (float)x.y;
    }
  for (int s = kMergePF; s < ns; ++s) {
    const h2 x = __builtin_bit_cast(h2, po[s * stride]);
    a0 += wgt[s] * (float)x.x;
    a1 += wgt[s] * (float)x.y;
  }
  const float o0 = L > 0.f ? a0 / L : 0.f, o1 = L > 0.f ? a1 / L : 0.f;
  if (!(__builtin_isfinite(o0) && __builtin_isfinite(o1))) atomicOr(fault, HSA_FAULT_RANGE);
  if (o_f32)
    *(float2*)((float*)O + (int64_t)qh * kD + 2 * lane) = make_float2(o0, o1);
  else
    ((uint32_t*)((u16*)O + (int64_t)qh * kD))[lane] =
        (uint32_t)__builtin_bit_cast(u16, (__bf16)o0) |
        ((uint32_t)__builtin_bit_cast(u16, (__bf16)o1) << 16);
  if (lane == 0 && lse) lse[qh] = (M + log2f(L)) * kLn2;
}

// One (query, head) per one-wave workgroup.
__global__ __launch_bounds__(64) void attn_merge_kernel(int H, int n_splits,
                                                        const u16* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        void* __restrict__ O, int o_f32,
                                                        float* __restrict__ lse, int* fault) {
  __shared__ float wgt[kMergeMaxSplits], wls[kMergeMaxSplits];
  merge_one(blockIdx.x, true, H, n_splits, part_o, part_ml, O, o_f32, lse, fault, wgt, wls);
}

// The merge with the decode cache upkeep of an HCA layer: two (query, head)
// waves per 128-thread workgroup, then one workgroup per request running the
// upkeep (the attention read each new token from its input and has finished
// with every page an fp8 re-encoding may rewrite).
__global__ __launch_bounds__(128) void attn_merge_upd_kernel(int n_qh, int H, int n_splits,
                                                             const u16* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             void* __restrict__ O, int o_f32,
                                                             float* __restrict__ lse, int* fault,
                                                             UpdateArgs upd) {
  const int n_merge = (n_qh + 1) / 2;
  if ((int)blockIdx.x >= n_merge) {
    decode_update_body<true, 16>(upd, blockIdx.x - n_merge, fault);
    return;
  }
  __shared__ float wgt[2][kMergeMaxSplits], wls[2][kMergeMaxSplits];
  const int wave = threadIdx.x >> 6;
  const int qh = blockIdx.x * 2 + wave;
  merge_one(qh, qh < n_qh, H, n_splits, part_o, part_ml, O, o_f32, lse, fault, wgt[wave],
            wls[wave]);
}

// ---------------------------------------------------------------- prefill HCA: query pairs

// Two consecutive prefill queries t0 and t1 = t0 + 1 of an HCA layer see the
// same compressed blocks (except possibly the last: n_vis(t0) <= n_vis(t1)) and
// windows that differ in one token at each end.  One workgroup walks the union
// of their entries once -- window tokens s(t0)..t1, then blocks 0..n_vis(t1)-1
// -- and every wave keeps two 16-head tiles, one per query, so each staged
// chunk and each K / V^T operand read from LDS feeds twice the MFMA work.
// Entries outside one query's own set are masked for that query only (in the
// few chunks that hold such entries).  bf16 caches, 64 heads per workgroup.
__global__ __launch_bounds__(256) void attn_pair_kernel(AttnArgs a) {
  constexpr int NT = 256, PPT = 4;
  unsigned bid = blockIdx.x;
  {
    unsigned per = gridDim.x / 8;
    bid = (bid % 8) * per + bid / 8;
  }
  const int hg = bid % a.n_hg;
  const int q0 = 2 * (int)(bid / a.n_hg);
  if (q0 >= a.n_q) return;
  const bool has1 = q0 + 1 < a.n_q;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  int r;
  int64_t t0;
  a.Q.get(q0, &r, &t0, a.fault);
  const int64_t t1 = has1 ? t0 + 1 : t0;
  const int64_t s0 = window_start(t0, a.n_win), s1 = window_start(t1, a.n_win);
  const int n_wu = (int)(t1 - s0 + 1);
  int64_t nv0 = n_visible(t0, a.m, a.n_win), nv1 = n_visible(t1, a.m, a.n_win);
  {
    int64_t ne = a.kc.n_entries[r];
    const int64_t ne2 = a.vc.n_entries[r];
    ne = ne < ne2 ? ne : ne2;
    ne = ne < 0 ? 0 : ne;
    if (nv1 > ne) {
      if (hg == 0 && tid == 0) atomicOr(a.fault, HSA_FAULT_ENTRIES);
      nv1 = ne;
      nv0 = nv0 < ne ? nv0 : ne;
    }
  }
  const int E = __builtin_amdgcn_readfirstlane(n_wu + (int)nv1);
  const int n_chunks = (E + 63) / 64;
  // tile 0 (t0): window entries 0..whi0, blocks < nv0; tile 1 (t1): window
  // entries wlo1..n_wu-1, blocks < nv1
  // uniform values, said so: the per-chunk mask test below stays a scalar branch
  const int whi0 = __builtin_amdgcn_readfirstlane((int)(t0 - s0));
  const int wlo1 = __builtin_amdgcn_readfirstlane((int)(s1 - s0));
  const int end0 = __builtin_amdgcn_readfirstlane(n_wu + (int)nv0);
  const int n_wuu = __builtin_amdgcn_readfirstlane(n_wu);

  // one LDS buffer for the K tile and then the V^T tile (fp16 bits, row pitch
  // 34 dwords: the 16 rows of a P V operand read on distinct bank pairs),
  // staged once every wave has read the K tile
  __shared__ __align__(16) u16 kv_lds[128 * 72];
  u16(*Ks)[136] = (u16(*)[136])kv_lds;
  u16(*Vt)[68] = (u16(*)[68])kv_lds;
  // dynamic LDS: row addresses of the union's entries (K, then V), sized by
  // the host for the longest union
  extern __shared__ __align__(16) int dyn_lds[];
  const uint8_t** rowk = (const uint8_t**)dyn_lds;
  const uint8_t** rowv = rowk + a.cps * 64;
  {
    const uint8_t* zero = (const uint8_t*)g_zero_row;
    // n_wu <= n_win + 1 rows from s0: at most one wrap of a ring whose
    // capacity the host checked (>= n_win + 1, or every position fits)
    const int64_t w0k = mod_nn(s0, a.wk.capacity), w0v = mod_nn(s0, a.wv.capacity);
    for (int j = tid; j < n_chunks * 64; j += NT) {
      const uint8_t *pk = zero, *pv = zero;
      if (j < n_wu) {
        pk = a.wk.data + ((int64_t)r * a.wk.capacity + ring_slot(w0k, j, a.wk.capacity)) * (kD * 2);
        pv = a.wv.data + ((int64_t)r * a.wv.capacity + ring_slot(w0v, j, a.wv.capacity)) * (kD * 2);
      } else if (j < E) {
        const int64_t b = j - n_wu;
        const int pgk = a.kc.page_of(r, b, a.fault), pgv = a.vc.page_of(r, b, a.fault);
        if (pgk >= 0) pk = a.kc.data + ((int64_t)pgk * kPage + (b & 63)) * (kD * 2);
        if (pgv >= 0) pv = a.vc.data + ((int64_t)pgv * kPage + (b & 63)) * (kD * 2);
      }
      rowk[j] = pk;
      rowv[j] = pv;
    }
  }
  const int head = hg * 64 + wave * 16 + col;
  bf16x8 qb[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = has1 ? q0 + j : q0;
    const bf16x8* qp = (const bf16x8*)(a.q + ((int64_t)qi * a.H + head) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[j][ks] = qp[4 * ks + g];
  }
  __syncthreads();

  uint4 kraw[PPT], vraw[PPT];
  const int vpair = tid & 31;
  auto issue_k = [&](int c) {
    const int lo = c * 64;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      kraw[i] = gload16((uintptr_t)rowk[lo + (p >> 4)] + (p & 15) * 16);
    }
  };
  auto issue_v = [&](int c) {
    const int lo = c * 64;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int ev = 2 * vpair + (i & 1), cgv = (tid >> 5) + (NT / 32) * (i >> 1);
      vraw[i] = gload16((uintptr_t)rowv[lo + ev] + cgv * 16);
    }
  };

  float m_i[2] = {-1e30f, -1e30f};
  f32x4 oacc[2][8], osum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    osum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;

  auto stage_v = [&]() {
#pragma unroll
    for (int j = 0; j < PPT / 2; ++j) {
      const int cgv = (tid >> 5) + (NT / 32) * j;
      const uint4 v0 = v_piece_f16(vraw[2 * j], false, 1.f);
      const uint4 v1 = v_piece_f16(vraw[2 * j + 1], false, 1.f);
      const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
      uint32_t* vt = (uint32_t*)&Vt[cgv * 8][0] + vpair;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        vt[(2 * q2) * 34] = (a0[q2] & 0xFFFFu) | (a1[q2] << 16);
        vt[(2 * q2 + 1) * 34] = (a0[q2] >> 16) | (a1[q2] & 0xFFFF0000u);
      }
    }
  };

  if (n_chunks > 0) {
    issue_k(0);
    issue_v(0);
  }
  for (int c = 0; c < n_chunks; ++c) {
    const int e0 = c * 64;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      *(uint4*)&Ks[p >> 4][(p & 15) * 8] = kraw[i];
    }
    __syncthreads();
    if (c + 1 < n_chunks) issue_k(c + 1);

    // ---- S^T = K Q^T for both queries; each K operand read once
    f32x4 sacc[2][4];
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      sacc[0][et] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[1][et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 av = *(const bf16x8*)&Ks[et * 16 + col][ks * 32 + 8 * g];
        sacc[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[0][ks], sacc[0][et], 0, 0, 0);
        sacc[1][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[1][ks], sacc[1][et], 0, 0, 0);
      }
    }
    // ---- masks, only in chunks that hold an entry outside either query's set
    const bool clean = e0 >= wlo1 && e0 + 64 <= end0 &&
                       (whi0 == n_wuu - 1 || e0 > whi0 + 1 || e0 + 63 < whi0 + 1);
    if (__builtin_expect(!clean, 0)) {
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = e0 + et * 16 + 4 * g + i;
          const bool ok0 = e < n_wu ? e <= whi0 : e < end0;
          const bool ok1 = e < n_wu ? e >= wlo1 : e < E;
          if (!ok0) sacc[0][et][i] = -INFINITY;
          if (!ok1) sacc[1][et][i] = -INFINITY;
        }
    }
    // ---- online softmax per query tile, then O^T += V^T P^T with shared V reads
    uint32_t pw[2][2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[j][et][i]);
      mx *= a.scale_log2;
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_i[j], mx);
      const float alpha = ex2(m_i[j] - m_new);
      m_i[j] = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[j][dt] *= alpha;
        osum[j] *= alpha;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          pw[j][h][i / 2] = pack_f16(ex2(__builtin_fmaf(sacc[j][2 * h][i], a.scale_log2, -m_new)),
                                     ex2(__builtin_fmaf(sacc[j][2 * h][i + 1], a.scale_log2, -m_new)));
          pw[j][h][2 + i / 2] =
              pack_f16(ex2(__builtin_fmaf(sacc[j][2 * h + 1][i], a.scale_log2, -m_new)),
                       ex2(__builtin_fmaf(sacc[j][2 * h + 1][i + 1], a.scale_log2, -m_new)));
        }
    }
    __syncthreads();   // every wave has read the K tile
    stage_v();
    __syncthreads();
    if (c + 1 < n_chunks) issue_v(c + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f16x8 pb0 = __builtin_bit_cast(f16x8, make_uint4(pw[0][h][0], pw[0][h][1], pw[0][h][2], pw[0][h][3]));
      const f16x8 pb1 = __builtin_bit_cast(f16x8, make_uint4(pw[1][h][0], pw[1][h][1], pw[1][h][2], pw[1][h][3]));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u16* vr = &Vt[16 * dt + col][0];
        const uint2 lo = *(const uint2*)(vr + 32 * h + 4 * g);
        const uint2 hi = *(const uint2*)(vr + 32 * h + 16 + 4 * g);
        const f16x8 av = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb0, oacc[0][dt], 0, 0, 0);
        oacc[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb1, oacc[1][dt], 0, 0, 0);
      }
      osum[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb0, osum[0], 0, 0, 0);
      osum[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb1, osum[1], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[16dt + 4g + i][head] of each query
  check_finite(oacc[0], a.fault);
  check_finite(oacc[1], a.fault);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j == 1 && !has1) break;
    const int qi = q0 + j;
    const float l = osum[j][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t o0 = ((int64_t)qi * a.H + head) * kD;
    if (a.o_f32) {
      float* orow = (float*)a.O + o0;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(orow + 16 * dt + 4 * g) = oacc[j][dt] * inv;
    } else {
      u16* orow = (u16*)a.O + o0;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(u16, (__bf16)(oacc[j][dt][i] * inv));
        *(uint2*)(orow + 16 * dt + 4 * g) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
    if (g == 0 && a.lse) a.lse[(int64_t)qi * a.H + head] = (m_i[j] + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------- host side

struct AttnPlan {
  int nw, n_hg, n_splits, cps;
};

// Listed (decode) queries: a query's entries are cut into splits of a fixed
// number of 64-entry chunks that depends only on the layer, never on the
// batch.  A request's partial results, and so its output bit for bit, are
// then the same alone or in any batch: splits past its own entries are empty
// and add exact zeros in the merge, which sums splits in a fixed order.
// CSA: a query has at most c = ceil((n_win + k) / 64) chunks; rows of up to 12
// chunks (k = 512 with the 128-token window: 10) go in pairs, longer rows one
// chunk per split (k = 1024: 18 splits, so that a batch of 4 still spreads
// over the chip), and never more than 32 splits.  HCA: 3 chunks per split (a
// batch of 4 at 1M tokens: 176 workgroups, one per CU with a chain of three
// chunks; 4 chunks left 124 CUs idle behind a longer chain, and 2 chunks make
// 260 workgroups, so that four CUs run two and set the kernel's time).
int attn_decode_cps(int k, int n_win) {
  if (k <= 0) return 3;
  const int chunks = (n_win + k + 63) / 64;
  if (chunks <= 12) return 2;
  return (chunks + 31) / 32;
}

static AttnPlan plan(int n_q, int H, int64_t max_entries, bool span, int decode_cps,
                     bool sel = false) {
  AttnPlan p;
  (void)n_q;
  // decode with 128 heads: an HCA split (three chunks) takes one 8-wave
  // workgroup for every head, so its rows are gathered once (two 4-wave head
  // groups gathered them twice and needed more workgroups than CUs); a CSA
  // split (sel: one chunk at k = 1024) takes two 4-wave workgroups of 64
  // heads, which halves each CU's LDS operand reads per chunk and starts
  // sooner, for a second gather of each row (Pro step 80.2 -> 79.2 us)
  p.nw = (!span && !sel && H % 128 == 0) ? 8 : (H % 64 == 0) ? 4 : (H % 32 == 0) ? 2 : 1;
  p.n_hg = H / (16 * p.nw);
  const int64_t chunks = (max_entries + 63) / 64 > 0 ? (max_entries + 63) / 64 : 1;
  if (span) {
    // prefill: at most kMaxCps chunks per workgroup (one query's entries fit)
    const int64_t n = (chunks + kMaxCps - 1) / kMaxCps;
    p.cps = (int)((chunks + n - 1) / n);
  } else {
    p.cps = decode_cps;
    // rows longer than the merge takes (beyond the decode limits) widen the
    // splits and lose the batch invariance
    if ((chunks + p.cps - 1) / p.cps > kMergeMaxSplits)
      p.cps = (int)((chunks + kMergeMaxSplits - 1) / kMergeMaxSplits);
  }
  p.n_splits = (int)((chunks + p.cps - 1) / p.cps);
  return p;
}

size_t attn_ws_bytes(int n_q, int H, int64_t max_entries, bool span, int decode_cps) {
  AttnPlan p = plan(n_q, H, max_entries, span, decode_cps);
  if (p.n_splits == 1) return 0;
  const size_t slots = (size_t)n_q * p.n_splits * H;
  return ((slots * kD * sizeof(u16) + 255) & ~size_t(255)) +
         ((slots * 2 * sizeof(float) + 255) & ~size_t(255)) + 256;
}

hipError_t launch_attn(const hsa_queries& q, const void* Q, int H, const hsa_tokens& wk,
                       const hsa_tokens& wv, int n_win, const hsa_paged& kc,
                       const hsa_paged& vc, int m, const int32_t* idx, int k, float scale,
                       void* O, int o_dtype, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t s, const UpdateArgs* upd) {
  const bool span = q.req == nullptr && q.pos == nullptr;
  int64_t s_max = q.max_pos - n_win + 1 < 0 ? 0 : q.max_pos - n_win + 1;
  int64_t nv_max = (s_max + m - 1) / m;
  int64_t b2 = (q.max_pos + 1) / m;
  nv_max = nv_max < b2 ? nv_max : b2;
  int64_t max_entries = n_win + (k > 0 ? (nv_max < k ? nv_max : k) : nv_max);
  AttnPlan p = plan(q.n, H, max_entries, span, attn_decode_cps(k, n_win), k > 0);
  // the partials this launch writes must fit the workspace it was given
  if (attn_ws_bytes(q.n, H, max_entries, span, attn_decode_cps(k, n_win)) > ws_bytes)
    return hipErrorInvalidValue;
  AttnArgs a;
  a.Q = to_dev(q, kc.n_req);
  a.q = (const u16*)Q;
  a.H = H;
  a.wk = to_dev(wk);
  a.wv = to_dev(wv);
  a.n_win = n_win;
  a.kc = to_dev(kc);
  a.vc = to_dev(vc);
  a.m = m;
  a.idx = idx;
  a.k = k;
  a.scale_log2 = scale * kLog2e;
  a.O = O;
  a.o_f32 = o_dtype == HSA_FP32;
  a.lse = lse;
  a.part_o = (u16*)ws;
  const size_t slots = (size_t)q.n * p.n_splits * H;
  a.part_ml = (float*)((char*)ws + ((slots * kD * sizeof(u16) + 255) & ~size_t(255)));
  a.n_splits = p.n_splits;
  a.cps = p.cps;
  a.n_hg = p.n_hg;
  a.n_q = q.n;
  a.fault = fault_word();
  // CSA decode of single-token queries (request = query index): the page
  // tables go to LDS when both rows are short enough
  a.pt_lds = (!span && k > 0 && q.req == nullptr && p.nw >= 4 &&
              kc.pages_per_req <= kPtLdsMax && vc.pages_per_req <= kPtLdsMax) ? 1 : 0;
  a.knew = a.vnew = nullptr;
  a.ring_rows = INT64_MAX;
  // the decode upkeep (upd): after the attention, in the merge launch, when
  // the queries are split (the attention then reads each query's own token
  // from k_new / v_new); otherwise before it, on its own
  bool upd_in_merge = false;
  if (upd) {
    const int64_t rows_k = (int64_t)wk.n_req * wk.capacity, rows_v = (int64_t)wv.n_req * wv.capacity;
    const int64_t rows = rows_k > rows_v ? rows_k : rows_v;
    upd_in_merge = !span && p.n_splits > 1 && p.nw >= 4 && rows + q.n < INT32_MAX - 2;
    if (upd_in_merge) {
      a.knew = upd->k_new;
      a.vnew = upd->v_new;
      a.ring_rows = rows;
    } else {
      hipError_t e = launch_update(*upd, q.n, s);
      if (e != hipSuccess) return e;
    }
  }
  int64_t n_blocks = (int64_t)q.n * p.n_hg * p.n_splits;
  a.xcd = span ? 1 : 0;
  if (a.xcd) n_blocks = (n_blocks + 7) / 8 * 8;
  const bool f8 = kc.dtype != HSA_BF16;   // fp8, or a mixed K with an fp8 V
  const bool kmix = kc.dtype == HSA_FP8_BF16_ROPE;
  // prefill of an HCA layer: pairs of consecutive queries share one walk over
  // their entries (the union of two windows needs n_win + 1 raw tokens)
  const int64_t need_cap = q.max_pos + 1 < n_win + 1 ? q.max_pos + 1 : n_win + 1;
  if (span && k == 0 && !f8 && H % 64 == 0 && n_win + 1 + nv_max <= kMaxCps * 64 &&
      wk.capacity >= need_cap && wv.capacity >= need_cap) {
    a.n_hg = H / 64;
    a.n_splits = 1;
    a.cps = (int)((n_win + 1 + nv_max + 63) / 64);   // chunks of the longest union
    const int64_t nb = ((int64_t)(q.n + 1) / 2 * a.n_hg + 7) / 8 * 8;
    timed_launch(HSA_K_ATTN, attn_pair_kernel, dim3((unsigned)nb), dim3(256),
                 (unsigned)(2 * a.cps * 64 * sizeof(const uint8_t*)), s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)n_blocks);
  // dynamic LDS: the row ids of a split's entries, and -- decode -- the
  // prefetched top-k ids (a split's entries plus one window) or page ids
  const size_t row_bytes = f8 ? sizeof(int) : sizeof(const uint8_t*);
  const unsigned pre = (unsigned)(2 * p.cps * 64 * row_bytes) +
                       (span ? 0u : (unsigned)((p.cps * 64 + n_win + 2 * kPrePages) * sizeof(int))) +
                       (a.pt_lds ? (unsigned)((kc.pages_per_req + vc.pages_per_req) * sizeof(int)) : 0u);
  // prefill (many workgroups per CU help): one LDS buffer for the K and V^T
  // tiles; decode (few workgroups, latency first): two
  if (p.nw == 4 && span && !f8)
    timed_launch(HSA_K_ATTN, attn_kernel<4, false, true, false>, grid, dim3(256), pre, s, a);
  else if (p.nw == 8 && upd_in_merge)
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<8, true, false, true, true>
                      : f8 ? attn_kernel<8, true, false, false, true>
                           : attn_kernel<8, false, false, false, true>,
                 grid, dim3(512), pre, s, a);
  else if (p.nw == 8)
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<8, true, false, true>
                      : f8 ? attn_kernel<8, true, false, false> : attn_kernel<8, false, false, false>,
                 grid, dim3(512), pre, s, a);
  else if (p.nw == 4 && upd_in_merge)
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<4, true, false, true, true>
                      : f8 ? attn_kernel<4, true, false, false, true>
                           : attn_kernel<4, false, false, false, true>,
                 grid, dim3(256), pre, s, a);
  else if (p.nw == 4)
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<4, true, false, true>
                      : f8 ? attn_kernel<4, true, false, false> : attn_kernel<4, false, false, false>,
                 grid, dim3(256), pre, s, a);
  else if (p.nw == 2)
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<2, true, false, true>
                      : f8 ? attn_kernel<2, true, false, false> : attn_kernel<2, false, false, false>,
                 grid, dim3(128), pre, s, a);
  else
    timed_launch(HSA_K_ATTN,
                 kmix ? attn_kernel<1, true, false, true>
                      : f8 ? attn_kernel<1, true, false, false> : attn_kernel<1, false, false, false>,
                 grid, dim3(64), pre, s, a);
  if (p.n_splits > 1) {
    const int n_qh = q.n * H;
    if (upd_in_merge)
      attn_merge_upd_kernel<<<(unsigned)((n_qh + 1) / 2 + q.n), 128, 0, s>>>(
          n_qh, H, p.n_splits, a.part_o, a.part_ml, O, a.o_f32, lse, a.fault, *upd);
    else
      attn_merge_kernel<<<(unsigned)n_qh, 64, 0, s>>>(H, p.n_splits, a.part_o, a.part_ml, O,
                                                       a.o_f32, lse, a.fault);
  }
  return hipGetLastError();
}

}  // namespace hsa
