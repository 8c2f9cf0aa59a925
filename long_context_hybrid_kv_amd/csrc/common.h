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
constexpr int kRopeDim = 64;   // rotated channels: the last 64 of a key row or a query head

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

// ---------------------------------------------------------------- positional rotation
// Partial RoPE (group-reading wiki "DeepSeek-V4 深度研究剖析" §8 keeps these
// channels of the KV cache in bf16): the last kRopeDim channels of a key row or
// of a query head turn as adjacent pairs (d-64+2i, d-63+2i) by the angle p * f_i
// at position p, with f_i = theta^(-2i/64) held in fp32.  The angle, its cos and
// sin and the turn are float64 (each product rounded, then the sum: no fused
// multiply-add); the result is rounded once to bf16.
struct RopeTab {
  double f[kRopeDim / 2];   // f_i: the fp32 table's values
};
RopeTab make_rope_tab(double theta);   // host

// Channel `odd` of a pair (x, y) turned by the angle whose cos / sin are c / s.
__device__ __forceinline__ double rope_turn(double x, double y, double c, double s, bool odd) {
#pragma clang fp contract(off)
  return odd ? x * s + y * c : x * c - y * s;
}

// A bf16 pair (the even channel in the low half) turned by the angle whose
// cos / sin are c / s.
__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t w, double c, double s) {
  const double x = bf16_to_f32((u16)(w & 0xFFFFu)), y = bf16_to_f32((u16)(w >> 16));
  return (uint32_t)f64_to_bf16(rope_turn(x, y, c, s, false)) |
         ((uint32_t)f64_to_bf16(rope_turn(x, y, c, s, true)) << 16);
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
// OCP MX FP4 of n_rows rows of 64 bf16 channels (row r at src + 64 r; rows
// >= n_valid read as zeros) by the rule the key compressor applies: per
// 32-channel block the scale 2^x, x = floor(log2 amax) - 2 clamped to
// [-127, 127] (0 for a block of zeros), each value / 2^x to the nearest e2m1
// code (ties to even, saturating at +-6; the sign bit follows the value).
// One channel a thread: each wave takes whole rows (lanes 0..31 block 0,
// 32..63 block 1).  Codes go to codes[r][w], channel c in bits 4 (c % 8) of
// word c / 8 (the nibble order of a stored key); scale bytes x + 127 to
// sb[r][c / 32].  Every thread of the workgroup calls it; the caller
// synchronises before reading the arrays.  (The scaling is exact in fp32: a
// bf16 value times 2^-x lands in [2^-6, 8) or is 0.)
__device__ __forceinline__ void mx_fp4_rows(const u16* __restrict__ src, int n_rows, int n_valid,
                                            uint32_t (*codes)[8], uint8_t (*sb)[2]) {
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int r = threadIdx.x >> 6; r < n_rows; r += nw) {
    const float x = r < n_valid ? __uint_as_float((uint32_t)src[(int64_t)r * 64 + lane] << 16) : 0.f;
    float a = fabsf(x);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    int E;
    (void)frexpf(a, &E);                       // a = f * 2^E, f in [0.5, 1)
    int xs = a > 0.f ? E - 3 : 0;
    xs = xs < -127 ? -127 : (xs > 127 ? 127 : xs);
    const float y = x * ldexpf(1.f, -xs);
    const float m = fminf(fabsf(y), 6.f);
    // the grid's quantum is 0.5 below 2, 1 in [2, 4), 2 in [4, 6]: its
    // multiples, rounded to even, give the magnitude code directly
    const float n = __builtin_rintf(m * (m < 2.f ? 2.f : (m < 4.f ? 1.f : 0.5f)));
    const uint32_t mag = (uint32_t)n + (m < 2.f ? 0u : (m < 4.f ? 2u : 4u));
    uint32_t wd = ((__builtin_signbit(y) ? 8u : 0u) | mag) << (4 * (lane & 7));
    wd |= __shfl_xor(wd, 1);
    wd |= __shfl_xor(wd, 2);
    wd |= __shfl_xor(wd, 4);
    if ((lane & 7) == 0) codes[r][lane >> 3] = wd;
    if ((lane & 31) == 0) sb[r][lane >> 5] = (uint8_t)(xs + 127);
  }
}
typedef int i32x8 __attribute__((ext_vector_type(8)));
// sum over 128 channels of a x b for MX FP4 operands on the 16x16x128 scaled
// MFMA (A: lane l holds row l % 16, channels 32 (l / 16) .. +31, with its
// block's scale byte; B likewise for column l % 16); acc += that product
__device__ __forceinline__ f32x4 mfma_mx_fp4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb,
                                            f32x4 acc) {
  const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  f32x4 r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc, 4, 4, 0, (int)sa, 0,
                                                             (int)sb);
  // an MFMA needs every lane of the wave: the empty statement keeps the
  // compiler from sinking it into a branch that only some lanes take (where
  // its result is used)
  asm volatile("" : "+v"(r));
  return r;
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

// A zero the compiler cannot see through.  A uniform value loaded at an index
// offset by it stays in a vector register until readfirstlane() moves it to a
// scalar one: the compiler would otherwise make that move (and wait for the
// load) right after each load, a round trip per value.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
__device__ __forceinline__ int64_t readfirstlane64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---- wave-wide scans and reductions by DPP lane moves (no LDS round trip;
// every lane of the wave active).  A step moves x from the lane CTRL names
// (row shift or row broadcast) into the 16-lane rows ROW_MASK selects; lanes
// with no source lane, and rows not selected, receive the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROW_MASK, 0xf, false);
}

// inclusive scan of an associative op over the 64 lanes, on 32-bit words:
// within each row by shifts of 1, 2, 4 and 8 lanes, then the rows' results
// carried on by the broadcasts of lane 15 (into rows 1 and 3) and lane 31
// (into rows 2 and 3)
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_bits(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_move<0x111, 0xf>(x, id));   // row_shr:1
  x = op(x, dpp_move<0x112, 0xf>(x, id));   // row_shr:2
  x = op(x, dpp_move<0x114, 0xf>(x, id));   // row_shr:4
  x = op(x, dpp_move<0x118, 0xf>(x, id));   // row_shr:8
  x = op(x, dpp_move<0x142, 0xa>(x, id));   // row_bcast:15
  x = op(x, dpp_move<0x143, 0xc>(x, id));   // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  return wave_incl_bits(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// the value of lane `l` (l uniform) in every lane
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// reductions over the wave, the result in every lane
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) { return lane_value(wave_incl_sum(x), 63); }
__device__ __forceinline__ int wave_max_i32(int x) {
  const uint32_t r = wave_incl_bits((uint32_t)x, 0x80000000u,
                                    [](uint32_t a, uint32_t b) { return (uint32_t)max((int)a, (int)b); });
  return (int)lane_value(r, 63);
}
__device__ __forceinline__ float wave_max_f32(float x) {
  const uint32_t r = wave_incl_bits(__float_as_uint(x), __float_as_uint(-INFINITY), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float(lane_value(r, 63));
}
// (a float sum in the scan's order: lane 0 first within each row, then the
// rows in order -- fixed, independent of what the lanes hold)
__device__ __forceinline__ float wave_sum_f32(float x) {
  const uint32_t r = wave_incl_bits(__float_as_uint(x), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float(lane_value(r, 63));
}

// x / d and x % d for x >= 0, d >= 1.  A 64-bit division is a long scalar
// sequence that every wave of a workgroup repeats; a power-of-two divisor (the
// compression rates) is a shift, and operands below 2^32 take the 32-bit
// division.  The branches are uniform wherever the operands are.
__device__ __forceinline__ int64_t div_nn(int64_t x, int64_t d) {
  if ((d & (d - 1)) == 0) return x >> __builtin_ctzll((uint64_t)d);
  if (((uint64_t)x | (uint64_t)d) >> 32 == 0) return (int64_t)((uint32_t)x / (uint32_t)d);
  return x / d;
}
__device__ __forceinline__ int64_t mod_nn(int64_t x, int64_t d) { return x - div_nn(x, d) * d; }

__device__ __forceinline__ int64_t window_start(int64_t t, int n_win) {
  int64_t s = t - n_win + 1;
  return s < 0 ? 0 : s;
}
__device__ __forceinline__ int64_t n_visible(int64_t t, int m, int n_win) {
  int64_t s = window_start(t, n_win);
  int64_t a = div_nn(s + m - 1, m);
  int64_t b = div_nn(t + 1, m);
  return a < b ? a : b;
}

// ---------------------------------------------------------------- descriptors passed by value

constexpr int kStashRows = 128;   // stash rows per request (entry e at e mod 128)

struct Paged {
  uint8_t* data;
  float* scale;
  const int32_t* page_table;
  int32_t* n_entries;
  int32_t pages_per_req, n_pages, dim, dtype;
  double* stash;        // fp8 caches appended to: [n_req][kStashRows][dim] exact values, or null
  __device__ __forceinline__ double* stash_row(int r, int64_t e) const {
    return stash + ((int64_t)r * kStashRows + (e & (kStashRows - 1))) * dim;
  }
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
    return (u16*)data + ((int64_t)r * capacity + mod_nn(p, capacity)) * dim;
  }
};

struct Queries {
  const int32_t* req;
  const int64_t* pos;
  int32_t span_req;
  int64_t span_pos0;
  int64_t max_pos;
  int32_t n_req;        // requests the caches hold: listed ids must lie below it
  // request of query i; a listed id outside [0, n_req) reads request 0 and
  // raises HSA_FAULT_REQ
  __device__ __forceinline__ int req_of(int i, int* fault) const {
    if (!pos) return span_req;
    const int r = req ? req[i] : i;
    if ((unsigned)r >= (unsigned)n_req) {
      atomicOr(fault, HSA_FAULT_REQ);
      return 0;
    }
    return r;
  }
  // position of query i; a listed position outside [0, max_pos] is clamped
  // into it and raises HSA_FAULT_POS
  __device__ __forceinline__ int64_t pos_of(int i, int* fault) const {
    if (!pos) return span_pos0 + i;
    int64_t p = pos[i];
    if (p > max_pos || p < 0) {
      atomicOr(fault, HSA_FAULT_POS);
      p = p < 0 ? 0 : max_pos;
    }
    return p;
  }
  __device__ __forceinline__ void get(int i, int* r, int64_t* t, int* fault) const {
    *r = req_of(i, fault);
    *t = pos_of(i, fault);
  }
};

inline Paged to_dev(const hsa_paged& p) {
  return Paged{(uint8_t*)p.data, p.scale, p.page_table, p.n_entries, p.pages_per_req,
               p.n_pages, p.dim, p.dtype, p.stash};
}
inline Tokens to_dev(const hsa_tokens& t) { return Tokens{(uint8_t*)t.data, t.capacity, t.dim}; }
inline Queries to_dev(const hsa_queries& q, int n_req) {
  return Queries{q.req, q.pos, q.span_req, q.span_pos0, q.max_pos, n_req};
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

// rows of `heads` bf16 heads of `dim` channels: y = x with the last 64 channels
// of every head turned at the row's position (pos[i], or pos0 + i); y == x
// rotates in place, otherwise the other channels are copied
hipError_t launch_rope(const void* x, void* y, int64_t n_rows, int heads, int dim,
                       const int64_t* pos, int64_t pos0, double theta, hipStream_t s);

struct UpdateArgs;   // update.h

// group > 1 (listed queries): the draft scan's workspace shape
size_t indexer_ws_bytes(int n_q, int64_t max_nvis, int k, bool span, int group = 1);
int64_t indexer_max_blocks();   // longest visible-block row the decode indexer takes
// upd: when not null, the decode cache upkeep of request i runs in the scan
// launch (bf16 caches without RoPE: one extra workgroup per request), in the
// candidate selection launch (fp8 caches or RoPE, long rows) or in its own
// launch before the scan
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
// upd (decode, one token per request, listed queries = requests 0..n-1): the
// cache upkeep, run after the attention in the merge launch when the queries
// are split (the attention reads each query's own token from upd->k_new /
// v_new), else before it
hipError_t launch_attn(const hsa_queries& q, const void* Q, int H, const hsa_tokens& wk,
                       const hsa_tokens& wv, int n_win, const hsa_paged& kc,
                       const hsa_paged& vc, int m, const int32_t* idx, int k, float scale,
                       void* O, int o_dtype, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t s, const UpdateArgs* upd = nullptr);

// the decode upkeep kernel over prepared arguments (B requests, one token each)
hipError_t launch_update(const UpdateArgs& u, int B, hipStream_t s);
// n_entries of request b := keep[b] / m in every cache of the layer
hipError_t launch_decode_rewind(const hsa_layer& L, int B, const int64_t* keep, hipStream_t s);

// Q / q_rot: with L.rope_theta > 0 the upkeep writes the queries Q turned to q_rot
UpdateArgs make_update_args(const hsa_layer& L, const int64_t* pos, int64_t max_pos,
                            const void* k_new, const void* v_new, const void* kI_new,
                            const void* Q = nullptr, void* q_rot = nullptr);
// n_tok > 1: a draft of n_tok tokens per request (rows b * n_tok + i of the
// new-token arrays), appended in order; q_pos / q_req (or null) receive the
// request and position of each of the draft's queries
hipError_t launch_decode_update(const hsa_layer& L, int B, const int64_t* pos, int64_t max_pos,
                                const void* k_new, const void* v_new, const void* kI_new,
                                hipStream_t s, int n_tok = 1, int64_t* q_pos = nullptr,
                                int32_t* q_req = nullptr, const void* Q = nullptr,
                                void* q_rot = nullptr);

}  // namespace hsa
