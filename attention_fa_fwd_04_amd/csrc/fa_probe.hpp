// MFMA-only throughput probe: the attainable dense matrix-core rate of the
// part under a sustained load, against which the attention kernels' rates
// are also reported (the spec peaks assume the 2.4 GHz peak engine clock).
//
// Every wave runs four independent accumulator chains of one MFMA shape on
// operands drawn from a per-lane hash (finite, mixed signs), so the matrix
// pipe never waits on a dependency and the data is not constant.  Each wave
// writes one float derived from its accumulators so nothing is optimised
// away.
#pragma once

#include "fa_common.hpp"

#include <type_traits>

namespace fa {

enum ProbeKind { kProbeBf16 = 0, kProbeFp8 = 1, kProbeInt8 = 2 };

// Multiply-add operations (2 per MAC) of one instruction of each shape.
constexpr double probe_flops_per_mfma(int kind) {
  return kind == kProbeBf16 ? 2.0 * 32 * 32 * 16 : kind == kProbeFp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 32;
}

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ __launch_bounds__(256) void fa_mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = probe_hash(blockIdx.x * 256u + threadIdx.x);
  float sink = 0.f;
  if constexpr (KIND == kProbeBf16) {
    // bf16 values of magnitude in [2^-8, 2^-1), random sign and mantissa
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = probe_hash(seed + e);
      const uint16_t ba = (uint16_t)(((h & 1u) << 15) | ((119u + ((h >> 1) & 7u)) << 7) | ((h >> 4) & 0x7fu));
      const uint16_t bb = (uint16_t)((((h >> 11) & 1u) << 15) | ((119u + ((h >> 12) & 7u)) << 7) | ((h >> 15) & 0x7fu));
      a[e] = __builtin_bit_cast(__bf16, ba);
      b[e] = __builtin_bit_cast(__bf16, bb);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) sink += c0[i] + c1[i] + c2[i] + c3[i];
  } else if constexpr (KIND == kProbeFp8) {
    // e4m3 bytes with exponent field 4..9 (magnitudes 2^-3 .. 2^2), random sign and mantissa
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wa = 0, wb = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h = probe_hash(seed + 8 * e + k);
        wa |= (((h & 0x80u) | ((4u + (h >> 8) % 6u) << 3) | ((h >> 12) & 7u)) & 0xffu) << (8 * k);
        wb |= ((((h >> 16) & 0x80u) | ((4u + (h >> 20) % 6u) << 3) | ((h >> 26) & 7u)) & 0xffu) << (8 * k);
      }
      a[e] = (int)wa;
      b[e] = (int)wb;
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) sink += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    // int8 bytes with bit 6 clear; int32 sums may wrap, which does not matter here
    i32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = probe_hash(seed + e), g = probe_hash(seed + 97 + e);
      a[e] = (int)(h & 0xbfbfbfbfu);
      b[e] = (int)(g & 0xbfbfbfbfu);
    }
    i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) sink += (float)(c0[i] ^ c1[i] ^ c2[i] ^ c3[i]);
  }
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = sink;
}

// Conversion probe: the narrowing conversions of the attention kernels,
// applied to caller-given floats so their rounding can be checked bit by bit
// against the format definitions.  Each thread converts four consecutive
// inputs with the same helper the kernels use: e4m3x4 (kind 0, one byte
// each), pack2<__bf16> (kind 1) or pack2<_Float16> (kind 2, two bytes each).
enum CvtKind { kCvtE4m3 = 0, kCvtBf16 = 1, kCvtF16 = 2 };

template <int KIND>
__global__ __launch_bounds__(256) void fa_cvt_probe_kernel(const float* __restrict__ in, void* __restrict__ out,
                                                           int64_t quads) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= quads) return;
  const f32x4 x = *reinterpret_cast<const f32x4*>(in + 4 * i);
  if constexpr (KIND == kCvtE4m3) {
    reinterpret_cast<uint32_t*>(out)[i] = e4m3x4(x.x, x.y, x.z, x.w);
  } else {
    using T = typename std::conditional<KIND == kCvtBf16, __bf16, _Float16>::type;
    reinterpret_cast<u32x2*>(out)[i] = u32x2{pack2<T>(x.x, x.y), pack2<T>(x.z, x.w)};
  }
}

}  // namespace fa
