// Merge of two attention results over disjoint key sets of the same queries
// (K/V split along the sequence: the essay page "FlashAttention原理与工业实战",
// section 6.2, ring attention).  With lse the row log-sum-exp of each part:
//   lse = log(e^lse_a + e^lse_b),  O = O_a e^(lse_a - lse) + O_b e^(lse_b - lse)
// in fp32, the per-tile rescale of the online softmax applied once between
// the two parts.  HBM-bound: one 16-byte chunk of a row per lane, every lane
// of a row in the same wave (lanes_per_row is a power of two dividing 64),
// so a row's lse is read by all its lanes before lane 0 writes the result,
// and merging in place (o == o_a, lse == lse_a) is safe.
#pragma once

#include "fa_common.hpp"

namespace fa {

template <typename T>
__device__ __forceinline__ u32x4 lerp_chunk(u32x4 a, u32x4 b, float wa, float wb);

template <>
__device__ __forceinline__ u32x4 lerp_chunk<float>(u32x4 a, u32x4 b, float wa, float wb) {
  const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
  f32x4 r;
  r.x = __builtin_fmaf(x.x, wa, y.x * wb);
  r.y = __builtin_fmaf(x.y, wa, y.y * wb);
  r.z = __builtin_fmaf(x.z, wa, y.z * wb);
  r.w = __builtin_fmaf(x.w, wa, y.w * wb);
  return __builtin_bit_cast(u32x4, r);
}

template <typename T>
__device__ __forceinline__ u32x4 lerp_chunk(u32x4 a, u32x4 b, float wa, float wb) {
  const T* x = reinterpret_cast<const T*>(&a);
  const T* y = reinterpret_cast<const T*>(&b);
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = __builtin_fmaf((float)x[e], wa, (float)y[e] * wb);
  return pack_chunk<T>(r);
}

template <typename T>
__global__ __launch_bounds__(256) void fa_merge_kernel(
    const T* oa, const float* la, const T* ob, const float* lb, T* o, float* lse,
    int64_t rows, int row_bytes, int chunks_per_row, int lanes_per_row) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / lanes_per_row;
  const int c = (int)(g % lanes_per_row);
  if (row >= rows) return;
  const float a = la[row], b = lb[row];
  const float m = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(a - m), eb = expf(b - m);
    const float z = ea + eb;
    wa = ea / z;
    wb = eb / z;
    l = m + logf(z);
  }
  if (c < chunks_per_row) {
    const size_t off = (size_t)row * row_bytes + (size_t)c * 16;
    const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(oa) + off);
    const u32x4 y = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(ob) + off);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(o) + off) = lerp_chunk<T>(x, y, wa, wb);
  }
  if (lse != nullptr && c == 0) lse[row] = l;
}

}  // namespace fa
