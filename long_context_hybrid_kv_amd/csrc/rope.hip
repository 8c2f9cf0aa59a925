// Partial RoPE over rows of bf16 heads (the rotation is defined in common.h).
// The decode step turns its new keys and queries inside its own upkeep
// launch; this kernel serves prefill, which rotates the token rows before
// they are compressed and attended to.
//
// A workgroup takes kRopeRows rows: 256 threads first compute the cos / sin of
// the rows' 32 pair angles once (float64) into LDS, then walk every head's
// RoPE pairs as 32-bit words (consecutive threads, consecutive words of a
// head), and -- out of place -- copy the other channels in 16-byte pieces.
#include <cmath>

#include "common.h"

namespace hsa {

constexpr int kRopeRows = 8;   // rows per workgroup: 8 x 32 angles = 256 threads

RopeTab make_rope_tab(double theta) {
  RopeTab t;
  for (int i = 0; i < kRopeDim / 2; ++i)
    t.f[i] = (double)(float)std::pow(theta, -2.0 * i / kRopeDim);
  return t;
}

__global__ __launch_bounds__(256) void rope_kernel(const u16* x, u16* y, int64_t n_rows,
                                                   int heads, int dim,
                                                   const int64_t* __restrict__ pos, int64_t pos0,
                                                   RopeTab tab, int copy, int* fault) {
  __shared__ double cs[kRopeRows][kRopeDim / 2][2];
  const int64_t r0 = (int64_t)blockIdx.x * kRopeRows;
  {
    const int rr = threadIdx.x >> 5, i = threadIdx.x & 31;
    const int64_t row = r0 + rr;
    double c = 1.0, s = 0.0;
    if (row < n_rows) {
      int64_t p = pos ? pos[row] : pos0 + row;
      if (p < 0) {   // a listed position below 0: reported, the row is left as it is
        if (i == 0) atomicOr(fault, HSA_FAULT_POS);
        p = 0;
      }
      sincos((double)p * tab.f[i], &s, &c);
    }
    cs[rr][i][0] = c;
    cs[rr][i][1] = s;
  }
  __syncthreads();
  const int nr = n_rows - r0 < kRopeRows ? (int)(n_rows - r0) : kRopeRows;
  const int64_t row_len = (int64_t)heads * dim;
  const int pairs = heads * (kRopeDim / 2);   // RoPE words of a row
  for (int k = threadIdx.x; k < nr * pairs; k += blockDim.x) {
    const int rr = k / pairs, rem = k - rr * pairs, h = rem >> 5, i = rem & 31;
    const int64_t off = (r0 + rr) * row_len + (int64_t)h * dim + (dim - kRopeDim) + 2 * i;
    const uint32_t w = *(const uint32_t*)(x + off);
    *(uint32_t*)(y + off) = rope_pair_bf16(w, cs[rr][i][0], cs[rr][i][1]);
  }
  if (copy) {
    const int per_head = (dim - kRopeDim) / 8, pieces = heads * per_head;
    for (int k = threadIdx.x; k < nr * pieces; k += blockDim.x) {
      const int rr = k / pieces, rem = k - rr * pieces, h = rem / per_head, j = rem - h * per_head;
      const int64_t off = (r0 + rr) * row_len + (int64_t)h * dim + 8 * j;
      *(uint4*)(y + off) = *(const uint4*)(x + off);
    }
  }
}

hipError_t launch_rope(const void* x, void* y, int64_t n_rows, int heads, int dim,
                       const int64_t* pos, int64_t pos0, double theta, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t blocks = (n_rows + kRopeRows - 1) / kRopeRows;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  rope_kernel<<<(unsigned)blocks, 256, 0, s>>>((const u16*)x, (u16*)y, n_rows, heads, dim, pos,
                                                pos0, make_rope_tab(theta), x != y, fault_word());
  return hipGetLastError();
}

}  // namespace hsa
