// Decode-time cache upkeep of one request (group-reading wiki "DeepSeek-V4
// 深度研究剖析" §11.4: the raw window and the incomplete tail live in a state
// cache; every m tokens the tail becomes one compressed entry).
//
// Shared by the standalone upkeep kernel (HCA layers) and by the indexer scan
// kernel, which runs the upkeep of request b in one extra workgroup beside the
// scan of request b (CSA layers): the block that completes at position t is
// not visible to the query at t (it starts inside the window), so the scan
// never reads what the upkeep writes in the same launch.
#pragma once
#include "common.h"

namespace hsa {

struct UpdateArgs {
  Tokens rk, rv, ti;                 // K / V rings, indexer-key tail (CSA)
  const int64_t* pos;                // [B] position of the new token
  int64_t max_pos;
  const u16* k_new;                  // [B][128] bf16
  const u16* v_new;                  // [B][128]
  const u16* ki_new;                 // [B][64] (CSA)
  int m, csa;
  const float* ak;                   // [m][128] pooling weights
  const float* av;
  const float* ai;                   // [m][64] (CSA)
  Paged kc, vc, kic;
  int n_tok;                         // tokens per request (a draft: n_tok > 1)
  int64_t* q_pos;                    // [B * n_tok] positions of the draft's queries, or null
  int32_t* q_req;                    // [B * n_tok] their requests
};

// Pool block blk of channel c from the ring/tail; the newest token's own value
// is taken from the input rather than re-read from the ring.
__device__ __forceinline__ double pool_last(const Tokens& src, int r, int64_t blk, int m, int c,
                                            const float* __restrict__ alpha, int dim, u16 newest) {
  double acc = 0.0;
  for (int j = 0; j < m - 1; ++j)
    acc += (double)alpha[(int64_t)j * dim + c] * (double)bf16_to_f32(src.row(r, blk * m + j)[c]);
  acc += (double)alpha[(int64_t)(m - 1) * dim + c] * (double)bf16_to_f32(newest);
  return acc;
}

// Token i of request b (position pos[b] + i): write its K / V (and indexer
// key) into the rings; when it completes a block, pool the block and append it
// at n_entries.  Threads 0..127 of the workgroup carry the channels (a thread
// writes and pools its own channel, so tokens of one request are handled in
// order without cross-thread hand-off); every thread of the workgroup must call
// this (it synchronises the workgroup).
__device__ inline void decode_update_token(const UpdateArgs& u, int b, int i, int* fault) {
  const int c = threadIdx.x;
  const bool on = c < kD;
  __shared__ int ok;
  const int64_t p = u.pos[b] + i;
  const int64_t row = (int64_t)b * u.n_tok + i;   // the token's row in k_new / v_new / ki_new
  if (p < 0 || p > u.max_pos) {
    if (c == 0) atomicOr(fault, HSA_FAULT_POS);
    return;
  }
  u16 kn = 0, vn = 0, in = 0;
  if (on) {
    kn = u.k_new[row * kD + c];
    vn = u.v_new[row * kD + c];
    u.rk.row(b, p)[c] = kn;
    u.rv.row(b, p)[c] = vn;
  }
  if (u.csa && c < kDI) {
    in = u.ki_new[row * kDI + c];
    u.ti.row(b, p)[c] = in;
  }
  if ((p + 1) % u.m != 0) return;
  const int64_t blk = (p + 1) / u.m - 1;
  if (c == 0) {
    const int32_t ek = u.kc.n_entries[b], ev = u.vc.n_entries[b];
    const int32_t ei = u.csa ? u.kic.n_entries[b] : (int32_t)blk;
    ok = (ek == blk && ev == blk && ei == blk);
    if (!ok) atomicOr(fault, HSA_FAULT_ENTRIES);
  }
  __syncthreads();
  if (!ok) return;
  if (on) {
    const int pk = u.kc.page_of(b, blk, fault), pv = u.vc.page_of(b, blk, fault);
    if (pk >= 0)
      ((u16*)u.kc.row(pk, blk))[c] = f64_to_bf16(pool_last(u.rk, b, blk, u.m, c, u.ak, kD, kn));
    if (pv >= 0)
      ((u16*)u.vc.row(pv, blk))[c] = f64_to_bf16(pool_last(u.rv, b, blk, u.m, c, u.av, kD, vn));
  }
  if (u.csa && c < kDI) {
    const int pi = u.kic.page_of(b, blk, fault);
    if (pi >= 0)
      ((u16*)u.kic.row(pi, blk))[c] = f64_to_bf16(pool_last(u.ti, b, blk, u.m, c, u.ai, kDI, in));
  }
  __syncthreads();
  if (c == 0) {
    u.kc.n_entries[b] = (int32_t)(blk + 1);
    u.vc.n_entries[b] = (int32_t)(blk + 1);
    if (u.csa) u.kic.n_entries[b] = (int32_t)(blk + 1);
  }
}

// Request b's n_tok tokens in order, and (a draft) its queries' request and
// position for the selection and attention that follow.
__device__ inline void decode_update_body(const UpdateArgs& u, int b, int* fault) {
  for (int i = 0; i < u.n_tok; ++i) {
    decode_update_token(u, b, i, fault);
    __syncthreads();   // the next token's block check reuses the shared flag
  }
  if (u.q_pos)
    for (int i = threadIdx.x; i < u.n_tok; i += blockDim.x) {
      u.q_pos[(int64_t)b * u.n_tok + i] = u.pos[b] + i;
      u.q_req[(int64_t)b * u.n_tok + i] = b;
    }
}

}  // namespace hsa
