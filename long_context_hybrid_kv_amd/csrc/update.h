// Decode-time cache upkeep of one request (group-reading wiki "DeepSeek-V4
// 深度研究剖析" §11.4: the raw window and the incomplete tail live in a state
// cache; every m tokens the tail becomes one compressed entry).
//
// Shared by the standalone upkeep kernel (drafts, RoPE layers, short HCA
// rows), the indexer scan kernel (plain bf16 CSA layers: one extra workgroup
// per request beside its scan), the candidate selection kernel (CSA layers
// with fp8 caches or RoPE, long rows: extra workgroups beside the selection)
// and the attention's merge kernel (HCA layers: after the attention, which
// read the new token from its input).  The block that completes at position t
// is not visible to the query at t (it starts inside the window), so nothing
// in the same launch reads what the upkeep writes.
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
  // partial RoPE (rope_on; the full upkeep only): each new key is turned at
  // its position before it enters the ring, so a block pools turned keys, and
  // the queries q_in [B * n_tok][H][128] are written turned to q_out
  int rope_on;
  RopeTab rope;
  const u16* q_in;
  u16* q_out;
  int H;
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

// pool_last of the K and V rings together, with PB ring rows of each (and
// their weights) requested at once: the block's m - 1 older rows cost
// ceil((m - 1) / PB) memory round trips instead of one per row, while the
// float64 sums still run in slot order, so the values are pool_last's.
template <int PB>
__device__ __forceinline__ void pool_last_kv(const Tokens& rk, const Tokens& rv, int r,
                                             int64_t blk, int m, int c,
                                             const float* __restrict__ ak,
                                             const float* __restrict__ av, u16 kn, u16 vn,
                                             double* vk, double* vv) {
  double sk = 0.0, sv = 0.0;
  const int n = m - 1;
  for (int j0 = 0; j0 < n; j0 += PB) {
    u16 xk[PB], xv[PB];
    float wk[PB], wv[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int j = j0 + u < n ? j0 + u : n - 1;   // (clamped reads past the block are unused)
      xk[u] = rk.row(r, blk * m + j)[c];
      xv[u] = rv.row(r, blk * m + j)[c];
      wk[u] = ak[(int64_t)j * kD + c];
      wv[u] = av[(int64_t)j * kD + c];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u)
      if (j0 + u < n) {
        sk += (double)wk[u] * (double)bf16_to_f32(xk[u]);
        sv += (double)wv[u] * (double)bf16_to_f32(xv[u]);
      }
  }
  *vk = sk + (double)ak[(int64_t)n * kD + c] * (double)bf16_to_f32(kn);
  *vv = sv + (double)av[(int64_t)n * kD + c] * (double)bf16_to_f32(vn);
}

// Largest v over the workgroup (every thread calls it; red holds >= 16 doubles).
__device__ __forceinline__ double block_max(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  __syncthreads();   // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double m = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = fmax(m, red[i]);
  return m;
}

// Re-encode the page holding entries p0 .. ne-1 (p0 = the page's first entry,
// ne > p0) of request b of an fp8 K / V cache from its stash: scale = amax /
// 448 over those entries (the fp8 channels of a mixed K), codes = e4m3(value /
// scale), the RoPE channels of a mixed K as bf16.  Thread c < kD carries
// channel c; every thread of the workgroup calls it.  only_last: the caller
// knows the page already holds entries p0 .. ne-2 encoded with some scale; if
// the new scale equals it, only entry ne-1 is written.
__device__ inline void reencode_open_page(const Paged& pc, int b, int64_t ne, bool only_last,
                                          int* fault, double* red) {
  const int c = threadIdx.x;
  const bool on = c < kD;
  const int64_t p0 = (ne - 1) & ~int64_t(kPage - 1);
  const int pg = pc.page_of(b, p0, fault);
  const bool scaled = on && (pc.dtype == HSA_FP8_E4M3 || c < kD / 2);
  double amax = 0.0;
  if (scaled)
    for (int64_t e = p0; e < ne; ++e) amax = fmax(amax, fabs(pc.stash_row(b, e)[c]));
  const float old = pg >= 0 ? pc.scale[pg] : 0.f;   // read before thread 0 rewrites it
  amax = block_max(amax, red);
  if (pg < 0) return;
  const float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
  const int64_t e_lo = (only_last && sc == old) ? ne - 1 : p0;
  if (on) {
    for (int64_t e = e_lo; e < ne; ++e) {
      const double v = pc.stash_row(b, e)[c];
      uint8_t* row = pc.row(pg, e);
      if (pc.dtype == HSA_FP8_BF16_ROPE && c >= kD / 2)
        ((u16*)(row + kD / 2))[c - kD / 2] = f64_to_bf16(v);
      else
        row[c] = f64_to_e4m3(v / (double)sc);
    }
  }
  if (c == 0) pc.scale[pg] = sc;
}

// Append entry blk (pooled value v of channel c, threads c < kD) to request b
// of a compressed K or V cache: bf16 rounds it into its row; fp8 formats (F8
// only) keep the exact value in the stash and re-encode the open page.  Every
// thread of the workgroup calls it.
template <bool F8>
__device__ inline void append_kv(const Paged& pc, int b, int64_t blk, double v, int* fault,
                                 double* red) {
  const int c = threadIdx.x;
  if (!F8 || pc.dtype == HSA_BF16) {
    if (c < kD) {
      const int pg = pc.page_of(b, blk, fault);
      if (pg >= 0) ((u16*)pc.row(pg, blk))[c] = f64_to_bf16(v);
    }
    return;
  }
  if (c < kD) pc.stash_row(b, blk)[c] = v;
  reencode_open_page(pc, b, blk + 1, (blk & (kPage - 1)) != 0, fault, red);
}

// Token i of request b (position pos[b] + i): write its K / V (and indexer
// key) into the rings; when it completes a block, pool the block and append it
// at n_entries.  Threads 0..127 of the workgroup carry the channels (a thread
// writes and pools its own channel, so tokens of one request are handled in
// order without cross-thread hand-off); every thread of the workgroup must call
// this (it synchronises the workgroup).  F8: the full upkeep -- the K / V
// caches may be fp8, keys and queries may be turned (RoPE), the indexer keys
// may be fp4; the indexer scan launch, which carries the upkeep of plain bf16
// CSA layers, is compiled without it (its float64 page loops would raise the
// scan's registers).
// With RoPE (F8 path) the token's pair angles are computed here, once, and
// left in rcs[i] = (cos, sin) for the query at the same position; a position
// outside [0, max_pos] is clamped for that (the attention clamps it too).
// PB > 1: a completed block's older ring rows are read PB at a time
// (pool_last_kv); the launches that carry HCA layers' upkeep (m = 128) use it,
// the others keep the registers of the plain loop.
template <bool F8, int PB = 1>
__device__ inline void decode_update_token(const UpdateArgs& u, int b, int i, int* fault,
                                           double (*rcs)[2]) {
  const int c = threadIdx.x;
  const bool on = c < kD;
  __shared__ int ok;
  const int64_t p = u.pos[b] + i;
  const int64_t row = (int64_t)b * u.n_tok + i;   // the token's row in k_new / v_new / ki_new
  double sn = 0.0, cs = 1.0;
  if constexpr (F8) {
    if (u.rope_on && on && c >= kD - kRopeDim) {
      const int64_t pc = p < 0 ? 0 : (p > u.max_pos ? u.max_pos : p);
      const int fi = (c - (kD - kRopeDim)) >> 1;
      sincos((double)pc * u.rope.f[fi], &sn, &cs);
      if (!(c & 1)) {
        rcs[fi][0] = cs;
        rcs[fi][1] = sn;
      }
    }
  }
  if (p < 0 || p > u.max_pos) {
    if (c == 0) atomicOr(fault, HSA_FAULT_POS);
    return;
  }
  u16 kn = 0, vn = 0, in = 0;
  if (on) {
    kn = u.k_new[row * kD + c];
    vn = u.v_new[row * kD + c];
  }
  if constexpr (F8) {
    if (u.rope_on) {   // uniform: every lane takes part in the exchange
      const u16 other = (u16)__shfl_xor((int)kn, 1);
      if (on && c >= kD - kRopeDim) {
        const bool odd = c & 1;
        const double x = bf16_to_f32(odd ? other : kn), y = bf16_to_f32(odd ? kn : other);
        kn = f64_to_bf16(rope_turn(x, y, cs, sn, odd));
      }
    }
  }
  if (on) {
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
  {
    __shared__ double red[16];
    double vk = 0.0, vv = 0.0;
    if (on) {
      if constexpr (PB > 1) {
        pool_last_kv<PB>(u.rk, u.rv, b, blk, u.m, c, u.ak, u.av, kn, vn, &vk, &vv);
      } else {
        vk = pool_last(u.rk, b, blk, u.m, c, u.ak, kD, kn);
        vv = pool_last(u.rv, b, blk, u.m, c, u.av, kD, vn);
      }
    }
    append_kv<F8>(u.kc, b, blk, vk, fault, red);
    append_kv<F8>(u.vc, b, blk, vv, fault, red);
  }
  if (u.csa && c < kDI) {   // wave 0, every lane: channel c of the indexer key
    const int pi = u.kic.page_of(b, blk, fault);
    const double v = pool_last(u.ti, b, blk, u.m, c, u.ai, kDI, in);
    if (F8 && u.kic.dtype == HSA_FP4_E2M1_MX) {   // (fp4 keys take the full upkeep)
      // MX FP4 as the compressor stores it: the 32-channel block's amax over
      // its 32 lanes, the scale 2^x, x = floor(log2 amax) - 2, one e2m1 code a
      // lane, channel 2j in the low nibble of byte j
      double a = fabs(v);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) a = fmax(a, __shfl_xor(a, o));
      int E;
      (void)frexp(a, &E);                      // a = f * 2^E, f in [0.5, 1)
      int xs = a > 0.0 ? E - 3 : 0;
      xs = xs < -127 ? -127 : (xs > 127 ? 127 : xs);
      const uint32_t code = f64_to_e2m1(v * ldexp(1.0, -xs));
      const uint32_t odd = __shfl_xor(code, 1);
      if (pi >= 0 && (c & 1) == 0) u.kic.row(pi, blk)[c / 2] = (uint8_t)(code | (odd << 4));
      if (pi >= 0 && (c & 31) == 0)
        ((uint8_t*)u.kic.scale)[((int64_t)pi * kPage + (blk & 63)) * (kDI / 32) + c / 32] =
            (uint8_t)(xs + 127);
    } else if (pi >= 0) {
      ((u16*)u.kic.row(pi, blk))[c] = f64_to_bf16(v);
    }
  }
  __syncthreads();
  if (c == 0) {
    u.kc.n_entries[b] = (int32_t)(blk + 1);
    u.vc.n_entries[b] = (int32_t)(blk + 1);
    if (u.csa) u.kic.n_entries[b] = (int32_t)(blk + 1);
  }
}

// Query i of request b turned for the attention (F8 upkeep, rope_on) with the
// pair angles rcs the token step at the same position left in LDS: the
// query's 32-bit words, RoPE pairs turned and the other channels copied.
__device__ inline void rope_query(const UpdateArgs& u, int b, int i, const double (*rcs)[2]) {
  const int words = u.H * (kD / 2);
  const int64_t q0 = ((int64_t)b * u.n_tok + i) * u.H * kD;
  const uint32_t* src = (const uint32_t*)(u.q_in + q0);
  uint32_t* dst = (uint32_t*)(u.q_out + q0);
  for (int wi = threadIdx.x; wi < words; wi += blockDim.x) {
    const int f = (wi & (kD / 2 - 1)) - (kD - kRopeDim) / 2;   // pair of the word, if RoPE
    const uint32_t w = src[wi];
    dst[wi] = f >= 0 ? rope_pair_bf16(w, rcs[f][0], rcs[f][1]) : w;
  }
}

// Request b's n_tok tokens in order, and (a draft) its queries' request and
// position for the selection and attention that follow.
template <bool F8, int PB = 1>
__device__ inline void decode_update_body(const UpdateArgs& u, int b, int* fault) {
  __shared__ double rcs[kRopeDim / 2][2];   // RoPE: the current token's pair angles
  for (int i = 0; i < u.n_tok; ++i) {
    decode_update_token<F8, PB>(u, b, i, fault, rcs);
    __syncthreads();   // the next token's block check reuses the shared flag; rcs is complete
    if constexpr (F8) {
      if (u.q_out) {
        rope_query(u, b, i, rcs);
        __syncthreads();   // rcs is rewritten by the next token
      }
    }
  }
  if (u.q_pos)
    for (int i = threadIdx.x; i < u.n_tok; i += blockDim.x) {
      u.q_pos[(int64_t)b * u.n_tok + i] = u.pos[b] + i;
      u.q_req[(int64_t)b * u.n_tok + i] = b;
    }
}

}  // namespace hsa
