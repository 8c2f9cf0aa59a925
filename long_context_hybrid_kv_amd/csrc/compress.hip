// Block compression (CSA m = 4, HCA m = 128): softmax-weighted pooling of the m
// tokens of each block into one cache entry, stored as bf16 or as fp8 e4m3fn with
// one fp32 scale per 64-entry page.
//
// Pooling is accumulated in float64: each product of an fp32 weight and a bf16
// token is exact there, so the entry is rounded only once, into the cache type.
// The work is a streaming read of the tokens (HBM-bound); float64 FMA runs at
// the same rate as fp32 on gfx950, so it costs nothing here.
#include "update.h"

namespace hsa {

// alpha[j][c] = softmax_j(z[j][c]) in float64 (slot-order sum), rounded to fp32.
__global__ void pooling_weights_kernel(const float* __restrict__ z, int m, int dim,
                                       float* __restrict__ alpha) {
  int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= dim) return;
  float mx = z[c];
  for (int j = 1; j < m; ++j) mx = fmaxf(mx, z[(int64_t)j * dim + c]);
  double s = 0.0;
  for (int j = 0; j < m; ++j) s += exp((double)z[(int64_t)j * dim + c] - (double)mx);
  for (int j = 0; j < m; ++j)
    alpha[(int64_t)j * dim + c] = (float)(exp((double)z[(int64_t)j * dim + c] - (double)mx) / s);
}

hipError_t launch_pooling_weights(const float* z, int m, int dim, float* alpha, hipStream_t s) {
  pooling_weights_kernel<<<(dim + 63) / 64, 64, 0, s>>>(z, m, dim, alpha);
  return hipGetLastError();
}

// One workgroup per cache page touched by [first, first + n).  Each thread owns
// the (entry, channel) items idx = tid, tid + 256, ... of the page; consecutive
// threads read consecutive channels of a token row (coalesced).
// FMT: HSA_BF16, HSA_FP8_E4M3 (every channel fp8, page scale over all of
// them), HSA_FP8_BF16_ROPE (channels below dim/2 fp8 with a page scale over
// those channels, the RoPE channels above them bf16) or HSA_FP4_E2M1_MX (dim
// 64: e2m1 nibbles with a power-of-two scale per 32-channel block)
template <int FMT, int MAXV>
__global__ __launch_bounds__(256) void compress_kernel(Tokens x, int x_req, int req, int64_t first,
                                                       int64_t n, int m,
                                                       const float* __restrict__ alpha,
                                                       Paged out, int* fault) {
  const int dim = out.dim;
  const int64_t page_e0 = ((first >> 6) + blockIdx.x) << 6;
  const int64_t e_lo = page_e0 > first ? page_e0 : first;
  const int64_t e_hi = (page_e0 + kPage) < (first + n) ? (page_e0 + kPage) : (first + n);
  const int page = out.page_of(req, page_e0, fault);
  if (blockIdx.x == 0 && threadIdx.x == 0) out.n_entries[req] = (int32_t)(first + n);
  if (page < 0) return;

  const int items = kPage * dim;
  double vals[MAXV];
  double amax = 0.0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    int it = threadIdx.x + v * 256;
    vals[v] = 0.0;
    if (it >= items) continue;
    int64_t e = page_e0 + it / dim;
    int c = it % dim;
    if (e < e_lo || e >= e_hi) continue;
    double acc = 0.0;
    for (int j = 0; j < m; ++j) {
      const u16* row = x.row(x_req, e * m + j);
      acc += (double)alpha[(int64_t)j * dim + c] * (double)bf16_to_f32(row[c]);
    }
    vals[v] = acc;
    if (FMT != HSA_FP8_BF16_ROPE || c < dim / 2) amax = fmax(amax, fabs(acc));
  }
  if (FMT == HSA_FP4_E2M1_MX) {
    // dim 64: item it = entry * 64 + channel with it = tid + 256 v, so the 32
    // channels of a block are 32 consecutive lanes of one wave (all of the same
    // entry); the block's amax is a reduction over those lanes
    uint8_t* sb = (uint8_t*)out.scale;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int it = threadIdx.x + v * 256;
      double a = fabs(vals[v]);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) a = fmax(a, __shfl_xor(a, o));
      int E;
      (void)frexp(a, &E);                       // a = f * 2^E, f in [0.5, 1)
      int x = a > 0.0 ? E - 3 : 0;              // floor(log2 a) - 2
      x = x < -127 ? -127 : (x > 127 ? 127 : x);
      const uint32_t code = f64_to_e2m1(vals[v] * ldexp(1.0, -x));   // exact scaling
      const uint32_t hi = __shfl_xor(code, 1);   // the odd channel's code
      const int64_t e = page_e0 + it / dim;
      const int c = it % dim;
      if (it >= items || e < e_lo || e >= e_hi) continue;
      if ((c & 1) == 0) out.row(page, e)[c / 2] = (uint8_t)(code | (hi << 4));
      if ((c & 31) == 0) sb[((int64_t)page * kPage + (e & 63)) * (dim / 32) + c / 32] = (uint8_t)(x + 127);
    }
    return;
  }
  if (FMT == HSA_BF16) {
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      int it = threadIdx.x + v * 256;
      if (it >= items) continue;
      int64_t e = page_e0 + it / dim;
      if (e < e_lo || e >= e_hi) continue;
      ((u16*)out.row(page, e))[it % dim] = f64_to_bf16(vals[v]);
    }
    return;
  }
  // fp8: page scale = amax / 448 over the entries written by this call
  __shared__ double red[4];
  for (int o = 32; o > 0; o >>= 1) amax = fmax(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
  if (threadIdx.x == 0) out.scale[page] = sc;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    int it = threadIdx.x + v * 256;
    if (it >= items) continue;
    int64_t e = page_e0 + it / dim;
    if (e < e_lo || e >= e_hi) continue;
    const int c = it % dim;
    uint8_t* row = out.row(page, e);
    if (FMT == HSA_FP8_BF16_ROPE && c >= dim / 2)
      ((u16*)(row + dim / 2))[c - dim / 2] = f64_to_bf16(vals[v]);   // RoPE channel
    else
      row[c] = f64_to_e4m3(vals[v] / (double)sc);
  }
}

// ---------------------------------------------------------------- decode: cache upkeep

// Decode-time cache upkeep for B requests (one workgroup each); the CSA decode
// step runs the same upkeep inside the indexer scan launch instead.
__global__ __launch_bounds__(128) void decode_update_kernel(UpdateArgs u, int* fault) {
  decode_update_body(u, blockIdx.x, fault);
}

// Rewind after a draft: request b keeps tokens 0 .. keep[b] - 1, so each of its
// caches keeps the keep[b] / m blocks those tokens complete.  A request whose
// keep lies outside [0, (n_entries + 1) * m) of any cache (more blocks than the
// cache holds) is left as it is and raises a fault.
__global__ void decode_rewind_kernel(const int64_t* __restrict__ keep, int B, int m, Paged kc,
                                     Paged vc, Paged kic, int csa, int* fault) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t p = keep[b];
  if (p < 0) {
    atomicOr(fault, HSA_FAULT_POS);
    return;
  }
  const int64_t e = p / m;
  const bool ok = e <= kc.n_entries[b] && e <= vc.n_entries[b] && (!csa || e <= kic.n_entries[b]);
  if (!ok) {
    atomicOr(fault, HSA_FAULT_ENTRIES);
    return;
  }
  kc.n_entries[b] = (int32_t)e;
  vc.n_entries[b] = (int32_t)e;
  if (csa) kic.n_entries[b] = (int32_t)e;
}

hipError_t launch_decode_rewind(const hsa_layer& L, int B, const int64_t* keep, hipStream_t s) {
  const int csa = L.kind == HSA_LAYER_CSA;
  decode_rewind_kernel<<<(B + 255) / 256, 256, 0, s>>>(keep, B, L.m, to_dev(L.kc), to_dev(L.vc),
                                                       csa ? to_dev(L.kic) : Paged{}, csa,
                                                       fault_word());
  return hipGetLastError();
}

UpdateArgs make_update_args(const hsa_layer& L, const int64_t* pos, int64_t max_pos,
                            const void* k_new, const void* v_new, const void* kI_new) {
  const int csa = L.kind == HSA_LAYER_CSA;
  UpdateArgs u;
  u.rk = to_dev(L.ring_k);
  u.rv = to_dev(L.ring_v);
  u.ti = csa ? to_dev(L.tail_i) : Tokens{nullptr, 1, kDI};
  u.pos = pos;
  u.max_pos = max_pos;
  u.k_new = (const u16*)k_new;
  u.v_new = (const u16*)v_new;
  u.ki_new = (const u16*)kI_new;
  u.m = L.m;
  u.csa = csa;
  u.ak = L.alpha_k;
  u.av = L.alpha_v;
  u.ai = L.alpha_i;
  u.kc = to_dev(L.kc);
  u.vc = to_dev(L.vc);
  u.kic = csa ? to_dev(L.kic) : Paged{};
  u.n_tok = 1;
  u.q_pos = nullptr;
  u.q_req = nullptr;
  return u;
}

hipError_t launch_decode_update(const hsa_layer& L, int B, const int64_t* pos, int64_t max_pos,
                                const void* k_new, const void* v_new, const void* kI_new,
                                hipStream_t s, int n_tok, int64_t* q_pos, int32_t* q_req) {
  UpdateArgs u = make_update_args(L, pos, max_pos, k_new, v_new, kI_new);
  u.n_tok = n_tok;
  u.q_pos = q_pos;
  u.q_req = q_req;
  decode_update_kernel<<<B, 128, 0, s>>>(u, fault_word());
  return hipGetLastError();
}

hipError_t launch_compress(const hsa_tokens& x, int x_req, const hsa_paged& out, int req,
                           int64_t first, int64_t n, int m, const float* alpha, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t pages = ((first + n - 1) >> 6) - (first >> 6) + 1;
  Paged o = to_dev(out);
  Tokens t = to_dev(x);
  KernelTimer kt(HSA_K_COMPRESS, s);
  const unsigned g = (unsigned)pages;
  int* f = fault_word();
  if (out.dtype == HSA_FP4_E2M1_MX) {     // indexer keys: dim = kDI
    compress_kernel<HSA_FP4_E2M1_MX, 16><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  } else if (out.dtype == HSA_FP8_BF16_ROPE) {   // K caches: dim = kD
    compress_kernel<HSA_FP8_BF16_ROPE, 32><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  } else if (out.dtype == HSA_FP8_E4M3) {
    if (out.dim == kD)
      compress_kernel<HSA_FP8_E4M3, 32><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
    else
      compress_kernel<HSA_FP8_E4M3, 16><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  } else {
    if (out.dim == kD)
      compress_kernel<HSA_BF16, 32><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
    else
      compress_kernel<HSA_BF16, 16><<<g, 256, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  }
  return hipGetLastError();
}

}  // namespace hsa
