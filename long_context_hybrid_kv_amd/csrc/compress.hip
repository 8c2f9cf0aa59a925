// Block compression (CSA m = 4, HCA m = 128): softmax-weighted pooling of the m
// tokens of each block into one cache entry, stored as bf16 or as fp8 e4m3fn with
// one fp32 scale per 64-entry page.
//
// Pooling is accumulated in float64: each product of an fp32 weight and a bf16
// token is exact there, so the entry is rounded only once, into the cache type.
// The work is a streaming read of the tokens (HBM-bound): m float64 FMAs per
// 2-byte token value, far below gfx950's vector float64 rate (half its fp32
// rate) at the bandwidth the reads allow.
//
// Layout of the work: a lane pools two adjacent channels, so a wave reads one
// whole 256-byte token row per load instruction (dim 128; two 128-byte rows
// for dim 64).  Formats without a page-wide scale (bf16, fp4 with its
// 32-channel blocks) give each lane group a run of consecutive entries whose
// token rows are consecutive (one HCA entry, or 16 CSA entries: 64 rows),
// with the run's row loads in flight together and the pooling weights in LDS;
// fp8 formats, whose page scale depends on all 64 entries of a page, give each
// page one workgroup of 16 waves (4 entries each) and reduce the page amax in
// LDS.
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

// Pooled value (float64, slot order) of channels c and c + 1 of entry e: the
// entry's m token rows are consecutive positions e*m .. e*m+m-1 of request
// x_req (row = position mod capacity, wrapped without a division per row).
__device__ __forceinline__ void pool2(const Tokens& x, int x_req, int64_t e, int m,
                                      const float* __restrict__ alpha, int dim, int c,
                                      double* s0, double* s1) {
  const int64_t cap = x.capacity;
  int64_t p = (e * m) % cap;
  const uint32_t* base = (const uint32_t*)((const u16*)x.data + (int64_t)x_req * cap * dim + c);
  const int64_t stride = dim / 2;              // 32-bit words per row
  double a0 = 0.0, a1 = 0.0;
#pragma unroll 16
  for (int j = 0; j < m; ++j) {
    const uint32_t v = __builtin_nontemporal_load(base + p * stride);
    const float2 al = *(const float2*)(alpha + (int64_t)j * dim + c);
    // each product is exact in float64, so contraction into an FMA changes nothing
    a0 += (double)al.x * (double)__uint_as_float(v << 16);
    a1 += (double)al.y * (double)__uint_as_float(v & 0xFFFF0000u);
    p = p + 1 == cap ? 0 : p + 1;
  }
  *s0 = a0;
  *s1 = a1;
}

// Entries [first, first + n) without a page-wide scale: HSA_BF16 (dim 128 or
// 64) and HSA_FP4_E2M1_MX (dim 64, power-of-two scale per 32-channel block).
// A lane group (dim / 2 lanes, two channels per lane) pools a run of epr =
// max(1, RR / m) consecutive entries: their m * epr token rows are consecutive
// positions, read RR at a time with every token load of the batch in flight
// before the slot-order accumulation uses them (bf16, RR = 64: an HCA entry in
// two batches, sixteen CSA entries in one).  The pooling weights sit in LDS
// when they fit (m * dim <= kAlphaLds floats), else they are read from memory.
constexpr int kAlphaLds = 16384;
template <int FMT> constexpr int run_rows() { return FMT == HSA_FP4_E2M1_MX ? 16 : 64; }

template <int FMT>
__device__ __forceinline__ void store_entry(const Paged& out, int req, int64_t e, int c,
                                            double v0, double v1, int* fault) {
  const int page = out.page_of(req, e, fault);
  if (FMT == HSA_FP4_E2M1_MX) {
    // the 32-channel block of these channels spans 16 lanes: its amax, the
    // power-of-two scale 2^x, x = floor(log2 amax) - 2, then two e2m1 codes
    double a = fmax(fabs(v0), fabs(v1));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) a = fmax(a, __shfl_xor(a, o));
    int E;
    (void)frexp(a, &E);                        // a = f * 2^E, f in [0.5, 1)
    int xs = a > 0.0 ? E - 3 : 0;
    xs = xs < -127 ? -127 : (xs > 127 ? 127 : xs);
    const double inv = ldexp(1.0, -xs);        // exact scaling
    const uint32_t code = f64_to_e2m1(v0 * inv) | (f64_to_e2m1(v1 * inv) << 4);
    if (page < 0) return;
    out.row(page, e)[c / 2] = (uint8_t)code;
    if ((c & 31) == 0)
      ((uint8_t*)out.scale)[((int64_t)page * kPage + (e & 63)) * (out.dim / 32) + c / 32] =
          (uint8_t)(xs + 127);
    return;
  }
  if (page < 0) return;
  ((uint32_t*)out.row(page, e))[c / 2] = (uint32_t)f64_to_bf16(v0) | ((uint32_t)f64_to_bf16(v1) << 16);
}

template <int FMT, bool ALDS>
__global__ __launch_bounds__(256) void compress_rows_kernel(Tokens x, int x_req, int req,
                                                            int64_t first, int64_t n, int m,
                                                            const float* __restrict__ alpha,
                                                            Paged out, int* fault) {
  constexpr int kRunRows = run_rows<FMT>();
  extern __shared__ float s_alpha[];
  const int dim = out.dim;
  const float* al = ALDS ? s_alpha : alpha;
  const int lpe = dim / 2;                     // lanes per entry
  const int lane = threadIdx.x & 63;
  const int epr = m >= kRunRows ? 1 : kRunRows / m;
  const int per_wg = 256 / lpe;                // runs per workgroup
  const int64_t i0 = ((int64_t)blockIdx.x * per_wg + threadIdx.x / lpe) * epr;
  if (blockIdx.x == 0 && threadIdx.x == 0) out.n_entries[req] = (int32_t)(first + n);
  const int c = 2 * (lane % lpe);
  const int rows = i0 < n ? (int)(n - i0 < epr ? n - i0 : epr) * m : 0;
  const int64_t cap = x.capacity;
  const uint32_t* base = (const uint32_t*)((const u16*)x.data + (int64_t)x_req * cap * dim + c);
  const int64_t stride = dim / 2;              // 32-bit words per row
  int64_t p = ((first + i0) * m) % cap;        // ring row of the run's first token
  double a0 = 0.0, a1 = 0.0;
  int j = 0;                                   // slot of the next row
  int64_t e = first + i0;                      // entry of the next row
  uint32_t v[kRunRows];
  auto load_batch = [&](int r0) {
#pragma unroll
    for (int u = 0; u < kRunRows; ++u) {
      v[u] = r0 + u < rows ? __builtin_nontemporal_load(base + p * stride) : 0u;
      p = p + 1 == cap ? 0 : p + 1;
    }
  };
  load_batch(0);   // in flight while the weights are staged
  if constexpr (ALDS) {
    // 16-byte pieces, sixteen per thread in flight (the host checked the
    // weights' alignment; m * dim is a multiple of 4)
    const int n4 = m * dim / 4;
    const float4* a4 = (const float4*)alpha;
    for (int i0 = 0; i0 < n4; i0 += 256 * 16) {
      float4 t[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 256 + threadIdx.x;
        t[u] = i < n4 ? a4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 256 + threadIdx.x;
        if (i < n4) ((float4*)s_alpha)[i] = t[u];
      }
    }
    __syncthreads();
  }
  for (int r0 = 0; r0 < rows; r0 += kRunRows) {
    if (r0 > 0) load_batch(r0);
#pragma unroll
    for (int u = 0; u < kRunRows; ++u) {
      if (r0 + u < rows) {
        const float2 w = *(const float2*)(al + (int64_t)j * dim + c);
        // each product is exact in float64, so contraction into an FMA changes nothing
        a0 += (double)w.x * (double)__uint_as_float(v[u] << 16);
        a1 += (double)w.y * (double)__uint_as_float(v[u] & 0xFFFF0000u);
        if (++j == m) {
          store_entry<FMT>(out, req, e, c, a0, a1, fault);
          a0 = a1 = 0.0;
          j = 0;
          ++e;
        }
      }
    }
  }
}

// Entries of formats with a page-wide fp32 scale: HSA_FP8_E4M3 (dim 128 or 64;
// scale over every channel) and HSA_FP8_BF16_ROPE (dim 128; scale over the
// fp8 channels 0 .. dim/2-1, the RoPE channels stored bf16).  One 1024-thread
// workgroup per page touched by [first, first + n) (the host requires a page
// aligned first); each of its 16 waves pools 4 of the page's 64 entries (dim
// 128: one entry per wave at a time; dim 64: two).  The page scale
// = amax / 448 over the entries this call writes.
template <int FMT>
__global__ __launch_bounds__(1024) void compress_page_kernel(Tokens x, int x_req, int req,
                                                             int64_t first, int64_t n, int m,
                                                             const float* __restrict__ alpha,
                                                             Paged out, int* fault) {
  const int dim = out.dim;
  const int lpe = dim / 2;
  const int epw = 64 / lpe;                    // entries a wave pools at once
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t page_e0 = ((first >> 6) + blockIdx.x) << 6;
  const int64_t e_hi = (page_e0 + kPage) < (first + n) ? (page_e0 + kPage) : (first + n);
  const int page = out.page_of(req, page_e0, fault);
  if (blockIdx.x == 0 && threadIdx.x == 0) out.n_entries[req] = (int32_t)(first + n);
  const int c = 2 * (lane % lpe);
  constexpr int kMaxIt = 4;                    // 64 entries / 16 waves, dim 128
  double v[kMaxIt][2];
  double amax = 0.0;
  const int n_it = 4 / epw;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    v[it][0] = v[it][1] = 0.0;
    if (it >= n_it) continue;
    const int64_t e = page_e0 + (int64_t)(wv * 4 + it * epw + lane / lpe);
    if (e >= e_hi) continue;
    pool2(x, x_req, e, m, alpha, dim, c, &v[it][0], &v[it][1]);
    if (FMT != HSA_FP8_BF16_ROPE || c < dim / 2) amax = fmax(amax, fmax(fabs(v[it][0]), fabs(v[it][1])));
    // the last page written keeps its exact values for later appends
    if (out.stash && blockIdx.x == gridDim.x - 1)
      *(double2*)(out.stash_row(req, e) + c) = make_double2(v[it][0], v[it][1]);
  }
  __shared__ double red[16];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmax(amax, __shfl_xor(amax, o));
  if (lane == 0) red[wv] = amax;
  __syncthreads();
  amax = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmax(amax, red[i]);
  if (page < 0) return;
  const float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
  if (threadIdx.x == 0) out.scale[page] = sc;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    if (it >= n_it) continue;
    const int64_t e = page_e0 + (int64_t)(wv * 4 + it * epw + lane / lpe);
    if (e >= e_hi) continue;
    uint8_t* row = out.row(page, e);
    if (FMT == HSA_FP8_BF16_ROPE && c >= dim / 2) {       // RoPE channels: bf16
      ((uint32_t*)(row + dim / 2))[(c - dim / 2) / 2] =
          (uint32_t)f64_to_bf16(v[it][0]) | ((uint32_t)f64_to_bf16(v[it][1]) << 16);
    } else {
      ((uint16_t*)row)[c / 2] = (uint16_t)(f64_to_e4m3(v[it][0] / (double)sc) |
                                           ((uint32_t)f64_to_e4m3(v[it][1] / (double)sc) << 8));
    }
  }
}

// ---------------------------------------------------------------- decode: cache upkeep

// Decode-time cache upkeep for B requests (one workgroup each); the CSA decode
// step runs the same upkeep inside the indexer scan launch instead.
__global__ __launch_bounds__(128) void decode_update_kernel(UpdateArgs u, int* fault) {
  decode_update_body<true, 16>(u, blockIdx.x, fault);
}

// Rewind after a draft: request b keeps tokens 0 .. keep[b] - 1, so each of its
// caches keeps the keep[b] / m blocks those tokens complete.  A request whose
// keep lies outside [0, (n_entries + 1) * m) of any cache (more blocks than the
// cache holds) is left as it is and raises a fault.  fp8 K / V caches then
// re-encode the page still filling from the stash, with the scale of the
// entries they keep.  One 128-thread workgroup per request.
__global__ __launch_bounds__(128) void decode_rewind_kernel(const int64_t* __restrict__ keep,
                                                            int m, Paged kc, Paged vc, Paged kic,
                                                            int csa, int* fault) {
  const int b = blockIdx.x;
  __shared__ double red[16];
  const int64_t p = keep[b];
  const int64_t e = p < 0 ? 0 : p / m;
  const bool ok = p >= 0 && e <= kc.n_entries[b] && e <= vc.n_entries[b] &&
                  (!csa || e <= kic.n_entries[b]);
  __syncthreads();   // every thread has read the counts before thread 0 rewrites them
  if (!ok) {
    if (threadIdx.x == 0) atomicOr(fault, p < 0 ? HSA_FAULT_POS : HSA_FAULT_ENTRIES);
    return;
  }
  if (threadIdx.x == 0) {
    kc.n_entries[b] = (int32_t)e;
    vc.n_entries[b] = (int32_t)e;
    if (csa) kic.n_entries[b] = (int32_t)e;
  }
  if (e % kPage == 0) return;   // no page is partly filled
  if (kc.dtype != HSA_BF16) reencode_open_page(kc, b, e, false, fault, red);
  if (vc.dtype != HSA_BF16) reencode_open_page(vc, b, e, false, fault, red);
}

hipError_t launch_decode_rewind(const hsa_layer& L, int B, const int64_t* keep, hipStream_t s) {
  const int csa = L.kind == HSA_LAYER_CSA;
  decode_rewind_kernel<<<B, 128, 0, s>>>(keep, L.m, to_dev(L.kc), to_dev(L.vc),
                                         csa ? to_dev(L.kic) : Paged{}, csa, fault_word());
  return hipGetLastError();
}

UpdateArgs make_update_args(const hsa_layer& L, const int64_t* pos, int64_t max_pos,
                            const void* k_new, const void* v_new, const void* kI_new,
                            const void* Q, void* q_rot) {
  const int csa = L.kind == HSA_LAYER_CSA;
  UpdateArgs u{};
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
  u.rope_on = L.rope_theta > 0.0;
  if (u.rope_on) u.rope = make_rope_tab(L.rope_theta);
  u.q_in = (const u16*)Q;
  u.q_out = u.rope_on ? (u16*)q_rot : nullptr;
  u.H = L.H;
  return u;
}

hipError_t launch_update(const UpdateArgs& u, int B, hipStream_t s) {
  decode_update_kernel<<<B, 128, 0, s>>>(u, fault_word());
  return hipGetLastError();
}

hipError_t launch_decode_update(const hsa_layer& L, int B, const int64_t* pos, int64_t max_pos,
                                const void* k_new, const void* v_new, const void* kI_new,
                                hipStream_t s, int n_tok, int64_t* q_pos, int32_t* q_req,
                                const void* Q, void* q_rot) {
  UpdateArgs u = make_update_args(L, pos, max_pos, k_new, v_new, kI_new, Q, q_rot);
  u.n_tok = n_tok;
  u.q_pos = q_pos;
  u.q_req = q_req;
  decode_update_kernel<<<B, 128, 0, s>>>(u, fault_word());
  return hipGetLastError();
}

hipError_t launch_compress(const hsa_tokens& x, int x_req, const hsa_paged& out, int req,
                           int64_t first, int64_t n, int m, const float* alpha, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  Paged o = to_dev(out);
  Tokens t = to_dev(x);
  KernelTimer kt(HSA_K_COMPRESS, s);
  int* f = fault_word();
  if (out.dtype == HSA_FP8_E4M3 || out.dtype == HSA_FP8_BF16_ROPE) {
    const unsigned g = (unsigned)(((first + n - 1) >> 6) - (first >> 6) + 1);
    if (out.dtype == HSA_FP8_BF16_ROPE)
      compress_page_kernel<HSA_FP8_BF16_ROPE><<<g, 1024, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
    else
      compress_page_kernel<HSA_FP8_E4M3><<<g, 1024, 0, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  } else {
    const bool f4 = out.dtype == HSA_FP4_E2M1_MX;
    const int per_wg = 256 / (out.dim / 2);
    const int rr = f4 ? run_rows<HSA_FP4_E2M1_MX>() : run_rows<HSA_BF16>();
    const int epr = m >= rr ? 1 : rr / m;
    const int64_t runs = (n + epr - 1) / epr;
    const unsigned g = (unsigned)((runs + per_wg - 1) / per_wg);
    const bool alds = (int64_t)m * out.dim <= kAlphaLds && ((uintptr_t)alpha & 15) == 0;
    const unsigned lds = alds ? (unsigned)(m * out.dim * sizeof(float)) : 0u;
    if (f4)
      (alds ? compress_rows_kernel<HSA_FP4_E2M1_MX, true> : compress_rows_kernel<HSA_FP4_E2M1_MX, false>)
          <<<g, 256, lds, s>>>(t, x_req, req, first, n, m, alpha, o, f);
    else
      (alds ? compress_rows_kernel<HSA_BF16, true> : compress_rows_kernel<HSA_BF16, false>)
          <<<g, 256, lds, s>>>(t, x_req, req, first, n, m, alpha, o, f);
  }
  return hipGetLastError();
}

}  // namespace hsa
