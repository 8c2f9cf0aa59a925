// Internal helpers shared by the gfx950 kernels of libhsa_attn.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "hsa_attn.h"

namespace hsa {

constexpr int kD = 128;        // head dim of Q/K/V
constexpr int kDI = 64;        // indexer head dim
constexpr int kHI = 4;         // indexer heads
constexpr int kPage = 64;      // entries per cache page

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Nearest bf16 of a float64 in one step (ties to even): scale by a power of two
// so that the bf16 quantum becomes 1, round to integer (v_rndne_f64), scale back.
__device__ __forceinline__ u16 f64_to_bf16(double x) {
  int e;
  (void)frexp(x, &e);                       // |x| = f * 2^e, f in [0.5, 1)
  int ee = e - 1 < -126 ? -126 : e - 1;     // binade exponent (bf16 normal range)
  double q = ldexp(1.0, ee - 7);            // bf16 quantum in that binade
  double v = __builtin_rint(x / q) * q;     // exact scaling, one rounding
  return (u16)(__float_as_uint((float)v) >> 16);   // v is a bf16 value: exact
}

// float64 -> OCP fp8 e4m3fn code (ties to even; saturates at +-448; the sign
// bit follows x, so a negative value that rounds to zero gives 0x80).
__device__ __forceinline__ uint8_t f64_to_e4m3(double x) {
  uint32_t sign = __builtin_signbit(x) ? 0x80u : 0u;
  double a = fabs(x);
  a = a > 448.0 ? 448.0 : a;
  int e;
  (void)frexp(a, &e);
  int ee = e - 1 < -6 ? -6 : e - 1;
  double q = ldexp(1.0, ee - 3);
  double v = __builtin_rint(a / q) * q;    // representable magnitude, <= 448
  if (v == 0.0) return (uint8_t)sign;
  int e2;
  (void)frexp(v, &e2);
  int ev = e2 - 1;
  uint32_t code;
  if (ev < -6) {
    code = (uint32_t)(v * 512.0);                     // subnormal: v = mant * 2^-9
  } else {
    uint32_t mant = (uint32_t)((ldexp(v, -ev) - 1.0) * 8.0);
    code = ((uint32_t)(ev + 7) << 3) | mant;
  }
  return (uint8_t)(sign | code);
}

// float64 -> OCP MX e2m1 code (4 bits; ties to even; saturates at +-6; the sign
// bit follows x).  The grid's quantum is 0.5 below 2, 1 in [2, 4), 2 in [4, 6].
__device__ __forceinline__ uint32_t f64_to_e2m1(double x) {
  const uint32_t sign = __builtin_signbit(x) ? 8u : 0u;
  double a = fabs(x);
  a = a > 6.0 ? 6.0 : a;
  const double q = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
  const double v = __builtin_rint(a / q) * q;   // representable magnitude, <= 6
  const uint32_t mag = v < 2.0 ? (uint32_t)(2.0 * v)
                     : v < 4.0 ? (uint32_t)(v + 2.0) : (uint32_t)(4.0 + 0.5 * v);
  return sign | mag;
}

// e4m3fn code -> bf16 bits (exact: e4m3 values are bf16 values).  Normal
// codes keep exponent and fraction (re-biased 7 -> 127); the eight codes with
// a zero exponent field are subnormal multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  uint32_t s = (c & 0x80u) << 8;
  uint32_t em = c & 0x7Fu;
  uint32_t nrm = (em << 4) + (120u << 7);
  uint32_t sub = __float_as_uint((float)em * 0x1p-9f) >> 16;
  return s | (em < 8u ? sub : nrm);
}

// 8 e4m3fn codes (two 32-bit words, code 0 in the lowest byte) -> 8 bf16
// values, by the hardware converter: every e4m3 value is a float with at most
// 4 significant bits, so dropping the float's low 16 bits is exact.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// 8 e2m1 codes (one 32-bit word, channel 2j in the low nibble of byte j) times
// a power-of-two scale -> bf16x8, by the hardware converter (exact: such a
// product is a bf16 value for the scales a compressor writes).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16x8(uint32_t c, float scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
// an e8m0 scale byte (2^(byte - 127)) as a float
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b ? b << 23 : 0x00400000u);
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 c) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
  const f2 p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
  const f2 p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
  const f2 p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
  auto two = [](f2 v) {
    return (__float_as_uint(v.x) >> 16) | (__float_as_uint(v.y) & 0xFFFF0000u);
  };
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, (u4{two(p0), two(p1), two(p2), two(p3)}));
}

// Order-preserving 32-bit key of a float (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- method definitions

__device__ __forceinline__ int64_t window_start(int64_t t, int n_win) {
  int64_t s = t - n_win + 1;
  return s < 0 ? 0 : s;
}
__device__ __forceinline__ int64_t n_visible(int64_t t, int m, int n_win) {
  int64_t s = window_start(t, n_win);
  int64_t a = (s + m - 1) / m;
  int64_t b = (t + 1) / m;
  return a < b ? a : b;
}

// ---------------------------------------------------------------- descriptors passed by value

struct Paged {
  uint8_t* data;
  float* scale;
  const int32_t* page_table;
  int32_t* n_entries;
  int32_t pages_per_req, n_pages, dim, dtype;
  // bytes of one entry's row: dim elements, (HSA_FP8_BF16_ROPE) dim/2 fp8
  // codes followed by dim/2 bf16 channels, or (HSA_FP4_E2M1_MX) dim/2 bytes of
  // e2m1 nibbles
  __device__ __forceinline__ int row_bytes() const {
    return dtype == HSA_FP8_E4M3        ? dim
           : dtype == HSA_FP8_BF16_ROPE ? dim / 2 * 3
           : dtype == HSA_FP4_E2M1_MX   ? dim / 2
                                        : dim * 2;
  }
  // physical page of entry e of request r, or -1 (and a fault) if out of range
  __device__ __forceinline__ int page_of(int r, int64_t e, int* fault) const {
    int p = page_table[(int64_t)r * pages_per_req + (e >> 6)];
    if ((unsigned)p >= (unsigned)n_pages) {
      atomicOr(fault, HSA_FAULT_PAGE);
      return -1;
    }
    return p;
  }
  __device__ __forceinline__ uint8_t* row(int page, int64_t e) const {
    return data + ((int64_t)page * kPage + (e & 63)) * row_bytes();
  }
};

struct Tokens {
  uint8_t* data;        // bf16 rows
  int64_t capacity;
  int32_t dim;
  __device__ __forceinline__ u16* row(int r, int64_t p) const {
    return (u16*)data + ((int64_t)r * capacity + (p % capacity)) * dim;
  }
};

struct Queries {
  const int32_t* req;
  const int64_t* pos;
  int32_t span_req;
  int64_t span_pos0;
  int64_t max_pos;
  __device__ __forceinline__ void get(int i, int* r, int64_t* t, int* fault) const {
    if (pos) {
      *r = req ? req[i] : i;
      int64_t p = pos[i];
      if (p > max_pos || p < 0) {
        atomicOr(fault, HSA_FAULT_POS);
        p = p < 0 ? 0 : max_pos;
      }
      *t = p;
    } else {
      *r = span_req;
      *t = span_pos0 + i;
    }
  }
};

inline Paged to_dev(const hsa_paged& p) {
  return Paged{(uint8_t*)p.data, p.scale, p.page_table, p.n_entries, p.pages_per_req,
               p.n_pages, p.dim, p.dtype};
}
inline Tokens to_dev(const hsa_tokens& t) { return Tokens{(uint8_t*)t.data, t.capacity, t.dim}; }
inline Queries to_dev(const hsa_queries& q) {
  return Queries{q.req, q.pos, q.span_req, q.span_pos0, q.max_pos};
}

// ---------------------------------------------------------------- host-side launchers

int* fault_word();   // device pointer of the current device's fault word

// Records start/stop events around a launch when timing is enabled for `id`.
// With ext = true no events are recorded by the timer itself: the single
// kernel is launched by timed_launch with the pair handed to the dispatch,
// so the events carry that kernel's own start and end times.
struct KernelTimer {
  KernelTimer(int id, hipStream_t s, bool ext = false);
  ~KernelTimer();
  hipEvent_t start() const;
  hipEvent_t stop() const;
  int id_;
  hipStream_t s_;
  void* slot_;
  bool ext_;
};

// Launch one kernel; when timing is on for `id`, its dispatch timestamps go
// into the timer's event pair.
template <typename... KA, typename... A>
inline void timed_launch(int id, void (*kernel)(KA...), dim3 grid, dim3 block, unsigned lds,
                         hipStream_t s, A... args) {
  KernelTimer kt(id, s, true);
  if (kt.slot_)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, kt.start(), kt.stop(), 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

hipError_t launch_pooling_weights(const float* z, int m, int dim, float* alpha, hipStream_t s);
hipError_t launch_compress(const hsa_tokens& x, int x_req, const hsa_paged& out, int req,
                           int64_t first, int64_t n, int m, const float* alpha, hipStream_t s);

struct UpdateArgs;   // update.h

size_t indexer_ws_bytes(int n_q, int64_t max_nvis, int k, bool span);
int64_t indexer_max_blocks();   // longest visible-block row the decode indexer takes
// upd: when not null, the decode cache upkeep of request i runs in the scan
// launch (one extra workgroup per request)
hipError_t launch_indexer(const hsa_queries& q, const void* qI, const float* w,
                          const hsa_paged& kic, int m, int n_win, int k, int32_t* idx,
                          float* score, void* ws, size_t ws_bytes, hipStream_t s,
                          const UpdateArgs* upd = nullptr, int group = 1, bool s16 = false);
// group (2..4, listed queries, no upd): consecutive queries g*group ..
// g*group+group-1 belong to one request and share each pass over its keys.
// s16: the scores are rounded to bf16 before the selection (not with group > 1)

// decode: 64-entry chunks per split of a query (a layer constant, so a
// request's result does not depend on the batch it is in)
int attn_decode_cps(int k, int n_win);
size_t attn_ws_bytes(int n_q, int H, int64_t max_entries, bool span, int decode_cps);
hipError_t launch_attn(const hsa_queries& q, const void* Q, int H, const hsa_tokens& wk,
                       const hsa_tokens& wv, int n_win, const hsa_paged& kc,
                       const hsa_paged& vc, int m, const int32_t* idx, int k, float scale,
                       void* O, int o_dtype, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t s);

UpdateArgs make_update_args(const hsa_layer& L, const int64_t* pos, int64_t max_pos,
                            const void* k_new, const void* v_new, const void* kI_new);
// n_tok > 1: a draft of n_tok tokens per request (rows b * n_tok + i of the
// new-token arrays), appended in order; q_pos / q_req (or null) receive the
// request and position of each of the draft's queries
hipError_t launch_decode_update(const hsa_layer& L, int B, const int64_t* pos, int64_t max_pos,
                                const void* k_new, const void* v_new, const void* kI_new,
                                hipStream_t s, int n_tok = 1, int64_t* q_pos = nullptr,
                                int32_t* q_req = nullptr);

}  // namespace hsa
