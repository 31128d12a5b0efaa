// INT8-QK / FP8-PV attention variant (handbook page "算子加速：注意力、编译与融合",
// section "SageAttention": K smoothed by its mean, Q and K quantised to INT8
// so Q K^T runs on integer matrix cores, P and V in FP8).
//
// Three prepass launches and the main kernel, all on the caller's stream:
//   int8_stats      per (b,h, 512-token split): float64 partial sums of K and
//                   partial max |V| per channel (fixed order, no atomics)
//   int8_finalize   per (b,h): kmean = fp32(sum / N); V scale av/448 and 448/av
//   int8_quant      per (b,h, 64-token block) and per Q, K, V:
//                   Q / K: X = Q or fp32(K - kmean), a = max |X|, codes
//                   rint(fp32(X * fp32(127/a))) in [-127,127], scale fp32(a/127);
//                   V: e4m3(fp32(V * fp32(448/av))), written transposed as
//                   V^T[d][key] with the key order of each 64-key group
//                   permuted to match the P operand
//   fa_int8qk       the online-softmax loop: S = (Q8 K8^T) * sq * sk * scale
//                   from exact int32 sums; P against the exact running max
//                   (no lazy rescale: P <= 1 is what makes the x448 FP8 scale
//                   valid), rounded to e4m3 as 448 P; l sums the unrounded
//                   448 P; O = acc * sv / l.
// With Q smoothing (the same section's "Q and K minus their block means")
// the Q slice of int8_quant also takes each 64-token block's mean qbar
// (float64 sum over the block's rows, rounded once to float32) and quantises
// Q - qbar; one more launch, int8_comp, tabulates the compensation
// scale log2(e) qbar_g . (K_j - kmean) in float64, rounded to float32, per
// (b,h, block, key); the main loop adds the wave's block row to its scores.
#pragma once

#include "fa_common.hpp"
#include "fa.h"

namespace fa {

constexpr int kInt8Bc = 64;        // keys per tile of the online softmax
constexpr int kQBlock = 64;        // tokens per INT8 scale block
constexpr int kStatRows = 512;     // tokens per partial-statistics workgroup (at least)
constexpr int kMaxSplits = 1024;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets of the workspace regions (each 256-byte aligned).
struct Int8Layout {
  int npad;          // N rounded up to kQBlock
  int groups;        // npad / kQBlock
  int splits;        // token splits of the K-sum / V-absmax reduction
  int split_rows;    // tokens per split
  size_t q8, k8, v8t, sq, sk, sv, vmul, kmean, kpart, vpart;
  size_t qbar, comp;   // Q smoothing only (0 otherwise)
  size_t total;
};

// pv16: the INT8-QK / 16-bit-PV form keeps V^T in the input's 16-bit type.
// smooth: Q smoothing adds the block means and the compensation table.
inline Int8Layout int8qk_workspace_layout(int B, int H, int N, int D, bool pv16 = false, bool smooth = false) {
  Int8Layout L{};
  const size_t bh = (size_t)B * H;
  L.npad = (N + kQBlock - 1) / kQBlock * kQBlock;
  L.groups = L.npad / kQBlock;
  L.splits = (N + kStatRows - 1) / kStatRows;
  if (L.splits > kMaxSplits) L.splits = kMaxSplits;
  L.split_rows = (N + L.splits - 1) / L.splits;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  L.q8 = take(bh * L.npad * D);                    // int8 [BH, npad, D]
  L.k8 = take(bh * L.npad * D);                    // int8 [BH, npad, D]
  L.v8t = take(bh * (size_t)D * L.npad * (pv16 ? 2 : 1));   // e4m3 (or 16-bit) [BH, D, npad]
  L.sq = take(bh * L.groups * 4);                  // f32 [BH, groups]
  L.sk = take(bh * L.groups * 4);
  L.sv = take(bh * (size_t)D * 4);                 // f32 [BH, D]  av / 448
  L.vmul = take(bh * (size_t)D * 4);               // f32 [BH, D]  448 / av
  L.kmean = take(bh * (size_t)D * 4);              // f32 [BH, D]
  L.kpart = take(bh * (size_t)L.splits * D * 8);   // f64 [BH, splits, D]
  L.vpart = take(bh * (size_t)L.splits * D * 4);   // f32 [BH, splits, D]
  if (smooth) {
    L.qbar = take(bh * L.groups * (size_t)D * 4);  // f32 [BH, groups, D]
    L.comp = take(bh * L.groups * (size_t)L.npad * 4);   // f32 [BH, groups, npad], log2 units
  }
  L.total = off;
  return L;
}

// Position of key k (0..63) inside its 64-key group of V^T.  The P operand of
// the FP8 32x32x64 MFMA takes, from lane half h, the 32 scores it holds for
// the group in accumulator order: slot e = 16G + 4g + r is key 32G + 8g + 4h + r.
// V^T row d stores at position 32h + e the key that slot pairs with.
__host__ __device__ constexpr int v8_pos(int k) {
  return 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);
}

// ---------------------------------------------------------------- prepass

template <typename T, int D>
__global__ __launch_bounds__(256) void int8_stats_kernel(
    const T* __restrict__ K, const T* __restrict__ V, double* __restrict__ kpart,
    float* __restrict__ vpart, int N, int splits, int split_rows) {
  static_assert(D == 128 && sizeof(T) == 2, "16-bit inputs, D = 128");
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int RG = 256 / CH;                  // row groups
  __shared__ double ssum[RG][D];
  __shared__ float smax[RG][D];
  const int s = blockIdx.x, bh = blockIdx.y;
  const int c = threadIdx.x % CH, rg = threadIdx.x / CH;
  const size_t head = (size_t)bh * N * D;
  const int r0 = s * split_rows, r1 = min(N, r0 + split_rows);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0 + rg; r < r1; r += RG) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(K + head + (size_t)r * D + c * 8);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(V + head + (size_t)r * D + c * 8);
    const T* kt = reinterpret_cast<const T*>(&kv);
    const T* vt = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += (double)(float)kt[e];
      mx[e] = fmaxf(mx[e], fabsf((float)vt[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ssum[rg][c * 8 + e] = acc[e];
    smax[rg][c * 8 + e] = mx[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double t = 0;
    float m = 0;
    for (int g = 0; g < RG; ++g) {
      t += ssum[g][d];
      m = fmaxf(m, smax[g][d]);
    }
    kpart[((size_t)bh * splits + s) * D + d] = t;
    vpart[((size_t)bh * splits + s) * D + d] = m;
  }
}

template <int D>
__global__ __launch_bounds__(128) void int8_finalize_kernel(
    const double* __restrict__ kpart, const float* __restrict__ vpart, float* __restrict__ kmean,
    float* __restrict__ sv, float* __restrict__ vmul, int N, int splits) {
  const int bh = blockIdx.x, d = threadIdx.x;
  double t = 0;
  float m = 0;
  for (int s = 0; s < splits; ++s) {
    t += kpart[((size_t)bh * splits + s) * D + d];
    m = fmaxf(m, vpart[((size_t)bh * splits + s) * D + d]);
  }
  kmean[(size_t)bh * D + d] = (float)(t / (double)N);
  sv[(size_t)bh * D + d] = m > 0.f ? m / 448.f : 0.f;
  vmul[(size_t)bh * D + d] = m > 0.f ? 448.f / m : 0.f;
}

// One 64-token block of Q (isk == 0) or K - kmean (isk == 1), 256 threads.
// qbar != nullptr (Q only): Q smoothing.  The block's mean over its rows
// below N is summed in float64 (thread partials over its 4 rows, then 16
// partials per channel through LDS: 16 KB of dsum), rounded once to float32,
// stored, and subtracted (in float32) from those rows before quantising.
template <typename T, int D>
__device__ __forceinline__ void quant_qk_block(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ kmean,
    int8_t* __restrict__ q8, int8_t* __restrict__ k8, float* __restrict__ sq, float* __restrict__ sk,
    float* __restrict__ qbar, int N, int npad, int groups, int g, int bh, int isk, float* wmax, double* dsum) {
  static_assert(D == 128 && sizeof(T) == 2, "16-bit inputs, D = 128");
  constexpr int CH = D / 8;
  const T* X = (isk ? K : Q) + (size_t)bh * N * D;
  int8_t* X8 = (isk ? k8 : q8) + (size_t)bh * npad * D;
  const int t = threadIdx.x;
  float x[4][8];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int it = t + 256 * i;              // 64 rows x 16 chunks
    const int row = g * kQBlock + it / CH, c = it % CH;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row < N) raw = *reinterpret_cast<const u32x4*>(X + (size_t)row * D + c * 8);
    const T* v = reinterpret_cast<const T*>(&raw);
    float km[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (isk && row < N) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(kmean + (size_t)bh * D + c * 8);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(kmean + (size_t)bh * D + c * 8 + 4);
      km[0] = lo.x; km[1] = lo.y; km[2] = lo.z; km[3] = lo.w;
      km[4] = hi.x; km[5] = hi.y; km[6] = hi.z; km[7] = hi.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = (float)v[e] - km[e];
  }
  if (!isk && qbar != nullptr) {
    // this thread's rows t / 16 + 16 i, channels 8 (t % 16) + e
    const int c = t % CH;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double p = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) p += (double)x[i][e];         // rows past N hold 0
      dsum[t * 8 + e] = p;
    }
    __syncthreads();
    float* qb = wmax + 4;                     // 128 floats after the 4 wave maxima
    if (t < D) {
      const int cc = t / 8, e = t % 8;
      double tot = 0.0;
      for (int j = 0; j < 256 / CH; ++j) tot += dsum[(cc + CH * j) * 8 + e];
      const int rows = min(kQBlock, N - g * kQBlock);
      const float mean = (float)(tot / (double)rows);
      qb[t] = mean;
      qbar[((size_t)bh * groups + g) * D + t] = mean;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = g * kQBlock + (t + 256 * i) / CH;
      if (row < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] - qb[c * 8 + e];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[i][e]));
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((t & 63) == 0) wmax[t >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = a > 0.f ? 127.f / a : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int it = t + 256 * i;
    const int row = g * kQBlock + it / CH, c = it % CH;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = __builtin_rintf(x[i][e] * inv);
      r = fminf(fmaxf(r, -127.f), 127.f);
      w[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
    }
    *reinterpret_cast<u32x2*>(X8 + (size_t)row * D + c * 8) = u32x2{w[0], w[1]};
  }
  if (t == 0) (isk ? sk : sq)[(size_t)bh * groups + g] = a > 0.f ? a / 127.f : 0.f;
}

// One 64-token block of V -> e4m3, transposed into V^T[d][64g + v8_pos(k)]
// (keys >= N are zero), 256 threads.  Thread t converts keys 4m .. 4m+3
// (m = t % 16) of channels 8c .. 8c+7 (c = t / 16); v8_pos keeps 4
// consecutive keys in consecutive positions, so each channel's 4 bytes are
// one dword LDS store.  LDS rows of 72 bytes put the four channel groups of
// a wave (8 channels apart) in disjoint 16-bank ranges: the stores are
// conflict-free.
template <typename T, int D>
__device__ __forceinline__ void quant_v_block(
    const T* __restrict__ V, const float* __restrict__ vmul, uint8_t* __restrict__ v8t,
    int N, int npad, int g, int bh, uint8_t* tile) {
  static_assert(D == 128 && sizeof(T) == 2, "16-bit inputs, D = 128");
  constexpr int TS = kQBlock + 8;                // LDS row bytes (18 dwords)
  const int t = threadIdx.x;
  const T* Vh = V + (size_t)bh * N * D;
  const float* vm = vmul + (size_t)bh * D;
  const int m = t & 15, c8 = t >> 4;
  const f32x4 m0 = *reinterpret_cast<const f32x4*>(vm + 8 * c8);
  const f32x4 m1 = *reinterpret_cast<const f32x4*>(vm + 8 * c8 + 4);
  uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int row = g * kQBlock + 4 * m + kk;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row < N) raw = *reinterpret_cast<const u32x4*>(Vh + (size_t)row * D + 8 * c8);
    const T* v = reinterpret_cast<const T*>(&raw);
    const uint32_t lo = e4m3x4((float)v[0] * m0.x, (float)v[1] * m0.y, (float)v[2] * m0.z, (float)v[3] * m0.w);
    const uint32_t hi = e4m3x4((float)v[4] * m1.x, (float)v[5] * m1.y, (float)v[6] * m1.z, (float)v[7] * m1.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      word[e] |= ((lo >> (8 * e)) & 0xFFu) << (8 * kk);
      word[4 + e] |= ((hi >> (8 * e)) & 0xFFu) << (8 * kk);
    }
  }
  const int pos = v8_pos(4 * m);
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(tile + (8 * c8 + e) * TS + pos) = word[e];
  __syncthreads();
  // thread: channel d = t / 2, 32 positions (t % 2), four 8-byte LDS reads
  const int d = t >> 1, half = t & 1;
  u32x2 part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) part[i] = *reinterpret_cast<const u32x2*>(tile + d * TS + 32 * half + 8 * i);
  uint8_t* dst = v8t + ((size_t)bh * D + d) * npad + (size_t)g * kQBlock + 32 * half;
  *reinterpret_cast<u32x4*>(dst) = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
  *reinterpret_cast<u32x4*>(dst + 16) = u32x4{part[2].x, part[2].y, part[3].x, part[3].y};
}

// Position of key k (0..31) inside its 32-key block of the 16-bit V^T: the
// 32x32x16 P V MFMA takes, from lane half h and step cc, the 8 scores the
// lane holds for keys 16 cc + 4 h + {0..3} and 16 cc + 8 + 4 h + {0..3}; with
// key 8g + 4h + r stored at 16h + 4g + r those are 8 consecutive positions.
__host__ __device__ constexpr int v16_pos(int k) {
  return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3);
}

// One 64-token block of V (16-bit, unquantised), transposed into
// V^T[d][64 g + 32 (k >> 5) + v16_pos(k & 31)]; keys >= N are zero.
template <typename T, int D>
__device__ __forceinline__ void v16t_block(const T* __restrict__ V, T* __restrict__ vt, int N, int npad, int g,
                                           int bh, T* tile) {
  static_assert(D == 128 && sizeof(T) == 2, "16-bit inputs, D = 128");
  constexpr int TS = 64 + 8;                    // LDS row: 64 keys + pad (elements)
  const int t = threadIdx.x;
  const T* Vh = V + (size_t)bh * N * D;
  // thread: key k = t / 4, channels 32 * (t % 4) .. +31
  const int k = t >> 2, c0 = 32 * (t & 3);
  const int row = g * kQBlock + k;
  const int pos = 32 * (k >> 5) + v16_pos(k & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row < N) raw = *reinterpret_cast<const u32x4*>(Vh + (size_t)row * D + c0 + 8 * q);
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[(c0 + 8 * q + e) * TS + pos] = v[e];
  }
  __syncthreads();
  // thread: channel d = t / 2, 32 positions (t % 2)
  const int d = t >> 1, half = t & 1;
  T* dst = vt + ((size_t)bh * D + d) * npad + (size_t)g * kQBlock + 32 * half;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<u32x4*>(dst + 8 * c) = *reinterpret_cast<const u32x4*>(tile + d * TS + 32 * half + 8 * c);
}

// The quantisation launch: blockIdx = (64-token block, b * H + h, which):
// which 0 quantises Q, 1 K - kmean (per-block INT8 codes and scales), 2 V
// (e4m3 V^T, or the 16-bit V^T of the INT8-QK / 16-bit-PV form).
template <typename T, int D, bool PV16, bool SMOOTH>
__global__ __launch_bounds__(256) void int8_quant_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ kmean,
    const float* __restrict__ vmul, int8_t* __restrict__ q8, int8_t* __restrict__ k8, void* __restrict__ vt,
    float* __restrict__ sq, float* __restrict__ sk, float* __restrict__ qbar, int N, int npad, int groups) {
  constexpr int VT_BYTES = PV16 ? D * (64 + 8) * 2 : D * (kQBlock + 8);
  constexpr int SM_BYTES = 256 * 8 * 8 + 1024;   // float64 partials + wave maxima and block means
  constexpr int BYTES = (SMOOTH && SM_BYTES > VT_BYTES) ? SM_BYTES : VT_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[BYTES];
  const int g = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  if (which < 2) {
    quant_qk_block<T, D>(Q, K, kmean, q8, k8, sq, sk, SMOOTH ? qbar : nullptr, N, npad, groups, g, bh, which,
                         reinterpret_cast<float*>(lds + (SMOOTH ? 256 * 8 * 8 : 0)), reinterpret_cast<double*>(lds));
  } else if constexpr (PV16) {
    v16t_block<T, D>(V, static_cast<T*>(vt), N, npad, g, bh, reinterpret_cast<T*>(lds));
  } else {
    quant_v_block<T, D>(V, vmul, static_cast<uint8_t*>(vt), N, npad, g, bh, lds);
  }
}

// Q smoothing's compensation table, tile of 64 blocks x 64 keys per
// workgroup of 4 waves: comp[bh][g][j] = fp32(c2 * sum_d qbar[g][d] *
// Ks[j][d]) with Ks = fp32(K - kmean) (keys past N give 0) and c2 = scale *
// log2(e), the products and sums in float64 on the matrix cores
// (v_mfma_f64_16x16x4: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// and holds D[l / 16 + 4 r][l % 16] in its r-th double, as measured).  Wave w computes blocks
// 32 (w & 1) + 0..31 against keys 32 (w >> 1) + 0..31 as 2 x 2 MFMA tiles.
// qbar and Ks are staged in LDS as floats (exact in double), rows of 132 (a
// 64-lane read of 16 rows x 4 channels then hits 64 distinct banks), 66 KB
// per workgroup so that two share a CU and one's loads overlap the other's
// MFMAs.
template <typename T, int D>
__global__ __launch_bounds__(256) void int8_comp_kernel(
    const T* __restrict__ K, const float* __restrict__ kmean, const float* __restrict__ qbar,
    float* __restrict__ comp, int N, int npad, int groups, double c2) {
  static_assert(D == 128 && sizeof(T) == 2, "16-bit inputs, D = 128");
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  constexpr int RS = D + 4;
  __shared__ __attribute__((aligned(16))) float qs[64 * RS];   // block means
  __shared__ __attribute__((aligned(16))) float ks[64 * RS];   // K - kmean
  const int j0 = blockIdx.x * 64, g0 = blockIdx.y * 64, bh = blockIdx.z, t = threadIdx.x;
  const T* Kh = K + (size_t)bh * N * D;
  const float* km = kmean + (size_t)bh * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int it = t + 256 * i, r = it / 16, c = it % 16;
    float kv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (j0 + r < N) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(Kh + (size_t)(j0 + r) * D + 8 * c);
      const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] = (float)v[e] - km[8 * c + e];
    }
    float qv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (g0 + r < groups) {
      const float* src = qbar + ((size_t)bh * groups + g0 + r) * D + 8 * c;
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = src[e];
    }
    *reinterpret_cast<f32x4*>(ks + r * RS + 8 * c) = f32x4{kv[0], kv[1], kv[2], kv[3]};
    *reinterpret_cast<f32x4*>(ks + r * RS + 8 * c + 4) = f32x4{kv[4], kv[5], kv[6], kv[7]};
    *reinterpret_cast<f32x4*>(qs + r * RS + 8 * c) = f32x4{qv[0], qv[1], qv[2], qv[3]};
    *reinterpret_cast<f32x4*>(qs + r * RS + 8 * c + 4) = f32x4{qv[4], qv[5], qv[6], qv[7]};
  }
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int gb = 32 * (wave & 1), jb = 32 * (wave >> 1);
  f64x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int d0 = 0; d0 < D; d0 += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) av[x] = (double)qs[(gb + 16 * x + li) * RS + d0 + lk];
#pragma unroll
    for (int y = 0; y < 2; ++y) bv[y] = (double)ks[(jb + 16 * y + li) * RS + d0 + lk];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = g0 + gb + 16 * x + lk + 4 * r;
      if (g < groups) {
        float* dst = comp + ((size_t)bh * groups + g) * npad + j0 + jb + li;
#pragma unroll
        for (int y = 0; y < 2; ++y) dst[16 * y] = (float)(acc[x][y][r] * c2);
      }
    }
}

// The QK^T accumulators start at the bit pattern of the float 1.5 * 2^23.  An
// int8 dot product d over D = 128 channels has |d| <= 127 * 127 * 128 < 2^21,
// so the biased sum is the bit pattern of 1.5 * 2^23 + d, a float in
// [2^23, 2^24) where floats are spaced 1: one float subtraction recovers d
// exactly (cheaper than an int-to-float conversion), and the biased sums
// compare as integers in the order of d.
constexpr int kAccBias = 0x4B400000;
constexpr float kAccBiasF = 12582912.f;
__device__ __forceinline__ float unbias(int a) { return __builtin_bit_cast(float, a) - kAccBiasF; }

// ---------------------------------------------------------------- main kernel
//
// Same work split as fa_fwd_kernel: 4 waves x 32 query rows, S^T = K Q^T so a
// lane owns one query.  QK^T: v_mfma_i32_32x32x32_i8 (lane half h feeds the
// 16 bytes of chunk 2s + h of its row, as in the 16-bit kernel).  PV:
// v_mfma_f32_32x32x64_f8f6f4 on e4m3 operands, one instruction per 32
// channels per 64-key tile.  The int8 K tile and the e4m3 V^T tile reach
// LDS by buffer-load DMA into unpadded, chunk-swizzled rows (no staging
// registers or LDS stores; the operand reads are conflict-free).

// SQ: Q smoothing; comp holds the compensation table (log2 units), whose
// row for the wave's query block is added to every score (MASK is then
// none or a key length).
template <typename T, int MASK, bool SQ>
__global__ __launch_bounds__(256, 2) void fa_int8qk_kernel(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const float* __restrict__ comp, MaskArgs mask, T* __restrict__ O, float* __restrict__ LSE,
    int H, int N, int npad, int groups, int nqt, float c_log2) {
  constexpr int D = 128, BC = kInt8Bc, BR = 128, NT = 256;
  constexpr int KSTR = D;                       // int8 K row (128 bytes, chunks swizzled)
  constexpr int VSTR = BC;                      // e4m3 V^T row (64 keys, chunks swizzled)
  // SQ: the compensation rows of the workgroup's two query blocks travel with
  // each tile (one 1 KB DMA instruction: 2 rows x 64 keys used)
  constexpr int TBYTES = SQ ? 1024 : 0;
  constexpr int KBYTES = BC * KSTR, VBYTES = D * VSTR, BUF = KBYTES + VBYTES + TBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int b = bh / H, h = bh - b * H;

  int n_eff = N;
  if constexpr (MASK == kMaskLen) {
    const int L = reinterpret_cast<const int*>(mask.ptr)[b];
    n_eff = L < 0 ? 0 : (L > N ? N : L);
  }
  const int ntiles = (n_eff + BC - 1) / BC;

  const int8_t* Qh = q8 + (size_t)bh * npad * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k8 + (size_t)bh * npad * D, (uint32_t)npad * D);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v8t + (size_t)bh * D * npad, (uint32_t)D * npad);

  const int q_row = qt * BR + wave * 32 + ln;
  const bool q_ok = q_row < N;
  // rows past N are zero codes in the workspace (npad >= q_row + 1 within the tile)
  u32x4 qreg[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qreg[s] = *reinterpret_cast<const u32x4*>(Qh + (size_t)min(q_row, npad - 1) * D + (2 * s + lh) * 16);
  // every query of a wave lies in one 64-token scale block
  const float sq_w = sq[(size_t)bh * groups + min((qt * BR + wave * 32) / kQBlock, groups - 1)];
  const float* skh = sk + (size_t)bh * groups;
  // additive mask: this lane's query row (row 0 stands in for rows past N,
  // whose results are not stored)
  const float* mrow = nullptr;
  bool mvec = false;
  if constexpr (MASK == kMaskAdd) {
    mrow = reinterpret_cast<const float*>(mask.ptr) + b * mask.sb + h * mask.sh + (int64_t)(q_ok ? q_row : 0) * mask.sq;
    mvec = mask_rows_vec4(mask);
  }
  static_assert(!(SQ && MASK == kMaskAdd), "Q smoothing takes no additive mask");
  // SQ: lanes 0-15 of wave 0 fetch 64 keys of the compensation row of block
  // 2 qt, lanes 16-31 of block 2 qt + 1 (rows of npad floats); lanes 32-63,
  // and blocks past the last, read out of range, which gives zeros
  const uint32_t tbytes = SQ ? (uint32_t)groups * (uint32_t)npad * 4u : 0u;
  const __amdgpu_buffer_rsrc_t tr =
      make_rsrc(SQ ? static_cast<const void*>(comp + (size_t)bh * groups * npad) : static_cast<const void*>(k8), tbytes);
  const int trs = lane >> 4;
  const uint32_t toff = trs < 2 ? (uint32_t)(((2 * qt + trs) * npad + 4 * (lane & 15)) * 4) : kOobOffset;
  constexpr bool kRowTerm = SQ || MASK == kMaskAdd;   // a per-key term on every tile

  // Tiles reach LDS by buffer-load DMA (1 KB per instruction, two K and two
  // V instructions per wave and tile).  Rows are unpadded; the lane landing
  // at physical chunk c of row r fetches logical chunk c ^ swz(r), K:
  // swz = (r >> 1) & 7 (128-byte rows, two per 256-byte bank row), V^T:
  // swz = (r >> 2) & 3 (64-byte rows, four per bank row), so the 16 rows of
  // one 16-lane read phase fall in 16 distinct 16-byte bank groups.
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kb = wave * 2 + i;
    const int kr_ = kb * 8 + (lane >> 3), kc = lane & 7;
    koff[i] = (uint32_t)kr_ * D + (uint32_t)((kc ^ ((kr_ >> 1) & 7)) << 4);
    const int vr_ = kb * 16 + (lane >> 2), vc = lane & 3;
    voff[i] = (uint32_t)vr_ * (uint32_t)npad + (uint32_t)((vc ^ ((vr_ >> 2) & 3)) << 4);
  }
  auto dma_tile = [&](int j, int buf) {
    uint8_t* kb = smem + buf * BUF;
    uint8_t* vb = kb + KBYTES;
    const uint32_t krow = (uint32_t)(j * BC) * D, vcol = (uint32_t)(j * BC);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kb + (wave * 2 + i) * 1024), 16, koff[i] + krow, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vb + (wave * 2 + i) * 1024), 16, voff[i] + vcol, 0, 0, 0);
    }
    if constexpr (SQ) {
      if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tr, (lds_void*)(vb + VBYTES), 16, toff + (uint32_t)(j * BC) * 4u, 0, 0,
                                                 0);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;
  constexpr float kLog2_448 = 8.807354922057604f;

  auto step = [&](int j, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = j & 1;
    dma_tile(j + 1, buf ^ 1);                     // past the last tile: never read
    // additive mask values of this lane's 32 keys (keys past N read -inf),
    // loaded ahead of the MFMAs (measured no faster issued before the DMA)
    float mk[32];
    if constexpr (MASK == kMaskAdd) load_mask_tile<2>(mk, mrow, mask.sk, mvec, j * BC, n_eff, lh);
    const uint8_t* kb = smem + buf * BUF;
    const uint8_t* vb = kb + KBYTES;
    const int kv0 = j * BC;
    if constexpr (SQ) {
      // this wave's block row, staged with the tile: keys 32 G + 8 g + 4 lh + {0..3}
      const float* trow = reinterpret_cast<const float*>(vb + VBYTES) + 64 * (wave >> 1);
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(trow + 32 * G + 8 * g + 4 * lh);
          mk[16 * G + 4 * g] = x.x;
          mk[16 * G + 4 * g + 1] = x.y;
          mk[16 * G + 4 * g + 2] = x.z;
          mk[16 * G + 4 * g + 3] = x.w;
        }
      if (kv0 + BC > n_eff) {                     // the ragged last tile: keys past n_eff drop out
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int key = kv0 + 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * lh + (i & 3);
          if (key >= n_eff) mk[i] = -INFINITY;
        }
      }
    }
    const float c = sq_w * skh[j] * c_log2;       // one K scale block per tile

    i32x16 si[2];
#pragma unroll
    for (int G = 0; G < 2; ++G) {
#pragma unroll
      for (int i = 0; i < 16; ++i) si[G][i] = kAccBias;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int r = 32 * G + ln;
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + r * KSTR + ((((2 * st + lh) ^ ((r >> 1) & 7))) << 4));
        si[G] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                      __builtin_bit_cast(i32x4, qreg[st]), si[G], 0, 0, 0);
      }
    }
    // Full tiles: the row max is taken on the exact int32 sums and scaled once
    // (the tile's scale c is >= 0), and the scale is folded into the exp2 FMA.
    // The ragged last tile, and every tile under an additive mask, scales
    // first (then adds the mask) so dropped keys can be -inf.
    float s[32];
    float mx;
    if constexpr (MASKED) {
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + 32 * G + 8 * (i >> 2) + 4 * lh + (i & 3);
          if constexpr (SQ)                           // table already in log2 units; -inf past n_eff
            s[16 * G + i] = __builtin_fmaf(unbias(si[G][i]), c, mk[16 * G + i]);
          else if constexpr (MASK == kMaskAdd)
            s[16 * G + i] = __builtin_fmaf(unbias(si[G][i]), c, mk[16 * G + i] * kLog2e);
          else
            s[16 * G + i] = key < n_eff ? unbias(si[G][i]) * c : -INFINITY;
        }
      mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 32; ++i) mx = fmaxf(mx, s[i]);
    } else {
      int imx = si[0][0];
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          imx = max(imx, si[G][i]);
          s[16 * G + i] = unbias(si[G][i]);
        }
      mx = unbias(imx) * c;
    }
    mx = wave_max_halves_valu(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[p][i] *= alpha;
    }
    // 448 P = exp2(s - m + log2 448) <= 448; the FP8 operand is its e4m3 rounding
    const float moff = m_use - kLog2_448;
    auto pexp = [&](float x) {
      return MASKED ? __builtin_amdgcn_exp2f(x - moff) : __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -moff));
    };
    float psum = -0.f;                            // -0 + x == x: the first add folds away
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float p0 = pexp(s[i]);
      const float p1 = pexp(s[i + 1]);
      const float p2 = pexp(s[i + 2]);
      const float p3 = pexp(s[i + 3]);
      psum += (p0 + p1) + (p2 + p3);
      pk[i >> 2] = e4m3x4(p0, p1, p2, p3);
    }
    l_run += psum;
    const i32x8 bop = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                       (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 32 * p + ln, sw = (r >> 2) & 3;
      const uint8_t* vrow = vb + r * VSTR;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(vrow + (((2 * lh) ^ sw) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(vrow + (((2 * lh + 1) ^ sw) << 4));
      const i32x8 aop = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      acc[p] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc[p], 0, 0, 0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0): tile j + 1 landed
    __syncthreads();
  };

  dma_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if constexpr (kRowTerm) {
    for (int j = 0; j < ntiles; ++j) step(j, BoolTag<true>{});
  } else {
    const int nfull = n_eff / BC;
    for (int j = 0; j < nfull; ++j) step(j, BoolTag<false>{});
    if (nfull < ntiles) step(nfull, BoolTag<true>{});
  }

  const float l_tot = wave_sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = O + ((size_t)bh * N + q_row) * D;
    const float* svh = sv + (size_t)bh * D;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * p + 8 * g + 4 * lh;
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(svh + d0);
        store4<T>(orow + d0, acc[p][4 * g] * s4.x * inv, acc[p][4 * g + 1] * s4.y * inv,
                  acc[p][4 * g + 2] * s4.z * inv, acc[p][4 * g + 3] * s4.w * inv);
      }
    if (LSE != nullptr && lh == 0)
      LSE[(size_t)bh * N + q_row] =
          l_tot > 0.f ? (m_run + log2f(l_tot) - kLog2_448) * kLn2 : -INFINITY;
  }
}

// Prepass launches (statistics, quantisation, and with Q smoothing the
// compensation table) shared by both P V forms; returns the operands.
struct Int8Ops {
  int8_t *q8, *k8;
  void* vt;
  float *sq, *sk, *sv, *comp;
};

template <typename T, bool PV16>
Int8Ops int8_prepass(const void* q, const void* k, const void* v, int B, int H, int N, float scale, void* workspace,
                     const Int8Layout& L, bool smooth, hipStream_t st) {
  constexpr int D = 128;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Int8Ops op{reinterpret_cast<int8_t*>(ws + L.q8), reinterpret_cast<int8_t*>(ws + L.k8), ws + L.v8t,
             reinterpret_cast<float*>(ws + L.sq), reinterpret_cast<float*>(ws + L.sk),
             reinterpret_cast<float*>(ws + L.sv), smooth ? reinterpret_cast<float*>(ws + L.comp) : nullptr};
  float* vmul = reinterpret_cast<float*>(ws + L.vmul);
  float* kmean = reinterpret_cast<float*>(ws + L.kmean);
  double* kpart = reinterpret_cast<double*>(ws + L.kpart);
  float* vpart = reinterpret_cast<float*>(ws + L.vpart);
  float* qbar = smooth ? reinterpret_cast<float*>(ws + L.qbar) : nullptr;
  const T* Q = static_cast<const T*>(q);
  const T* K = static_cast<const T*>(k);
  const T* V = static_cast<const T*>(v);
  const int BH = B * H;
  hipLaunchKernelGGL((int8_stats_kernel<T, D>), dim3(L.splits, BH), dim3(256), 0, st, K, V, kpart, vpart, N, L.splits,
                     L.split_rows);
  hipLaunchKernelGGL((int8_finalize_kernel<D>), dim3(BH), dim3(D), 0, st, kpart, vpart, kmean, op.sv, vmul, N, L.splits);
  if (smooth) {
    hipLaunchKernelGGL((int8_quant_kernel<T, D, PV16, true>), dim3(L.groups, BH, 3), dim3(256), 0, st, Q, K, V,
                       kmean, vmul, op.q8, op.k8, op.vt, op.sq, op.sk, qbar, N, L.npad, L.groups);
    hipLaunchKernelGGL((int8_comp_kernel<T, D>), dim3(L.npad / 64, (L.groups + 63) / 64, BH), dim3(256), 0, st, K,
                       kmean, qbar, op.comp, N, L.npad, L.groups, (double)scale * 1.4426950408889634);
  } else {
    hipLaunchKernelGGL((int8_quant_kernel<T, D, PV16, false>), dim3(L.groups, BH, 3), dim3(256), 0, st, Q, K, V,
                       kmean, vmul, op.q8, op.k8, op.vt, op.sq, op.sk, nullptr, N, L.npad, L.groups);
  }
  return op;
}

template <typename T>
int launch_int8qk(const void* q, const void* k, const void* v, void* o, float* lse, int mask_kind, MaskArgs m,
                  int B, int H, int N, float scale, void* workspace, const Int8Layout& L, bool smooth,
                  hipStream_t st) {
  const Int8Ops op = int8_prepass<T, false>(q, k, v, B, H, N, scale, workspace, L, smooth, st);
  const int nqt = (N + 127) / 128;
  const int grid = B * H * nqt;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, op.q8, op.k8, static_cast<const uint8_t*>(op.vt), op.sq,
                       op.sk, op.sv, op.comp, m, static_cast<T*>(o), lse, H, N, L.npad, L.groups, nqt,
                       scale * kLog2e);
  };
  if (smooth) {
    if (mask_kind == kMaskLen) go(fa_int8qk_kernel<T, kMaskLen, true>);
    else go(fa_int8qk_kernel<T, kMaskNone, true>);
  } else if (mask_kind == kMaskLen) go(fa_int8qk_kernel<T, kMaskLen, false>);
  else if (mask_kind == kMaskAdd) go(fa_int8qk_kernel<T, kMaskAdd, false>);
  else go(fa_int8qk_kernel<T, kMaskNone, false>);
  return FA_OK;
}

}  // namespace fa
