// Attention forward for 16-bit types with D = 128, staging K and V tiles by
// LDS DMA (gfx950 `buffer_load_dwordx4 ... lds`).
//
// Same method and work split as fa_fwd_kernel (handbook page
// "算子加速：注意力、编译与融合", section "注意力：从 O(N²) 显存到分块": running row
// max and denominator, rescaled accumulator, only O written): waves of 32
// query rows compute S^T = K Q^T with 32x32 MFMAs so a lane owns one query,
// and accumulate O^T += V^T P^T.  What differs is how tiles reach LDS:
//
//  * K and V tiles go from global memory straight into LDS through the
//    buffer-load DMA path: no staging registers, no LDS write instructions,
//    no VALU work.  Each DMA instruction writes 64 lanes x 16 bytes to one
//    contiguous kilobyte of LDS, so rows are unpadded (256 bytes) and bank
//    conflicts are avoided by permuting the 16-byte chunks of each row: the
//    lane that lands at physical chunk c of row r fetches logical chunk
//    c ^ f(r) from global memory.  K uses f(r) = r & 15, which spreads the
//    16 rows one ds_read_b128 phase touches over all 16 chunk slots; V uses
//    the bit map v_swz below, which does the same for the transposing reads.
//  * V stays row-major in LDS.  The P V operand needs, per lane, consecutive
//    keys at one channel; ds_read_b64_tr_b16 provides exactly that: within
//    each 16-lane group, lane 4k + t fetches 4 channels (4t .. 4t+3) of key
//    k and the hardware hands lane j the 4 keys of channel j.  Two such reads
//    (keys 0-3 and 8-11 after the lane half's 4-key offset) make the 8-key
//    operand that pairs with the lane's own scores.
//
// With no staging registers or LDS write instructions, each wave's tile loop
// is only MFMA, LDS reads and the softmax arithmetic.  The library launches
// this kernel for additive masks: 8 waves (256 query rows) in step over
// 64-key tiles, four 16 KB buffers in LDS (without a score mask the same
// staging runs in the phase-alternating schedule of fa_fwd_pp.hpp).
#pragma once

#include "fa_common.hpp"
#include "fa_fwd_kernel.hpp"

namespace fa {

template <typename T, int BC, int NW>
struct DmaCfg {
  static constexpr int D = 128;
  static constexpr int ROW = 256;                 // bytes per K / V row in LDS
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;
  static constexpr int TILE = BC * ROW;           // bytes per K (or V) tile
  static constexpr int SB = BC / 32;
  static constexpr int QKS = 8;                   // MFMA steps over D
  static constexpr int PVB = 4;                   // 32-channel blocks of O^T
  static constexpr int DMA_PER_WAVE = TILE / 1024 / NW;   // 1 KB per DMA instruction
  static_assert(sizeof(T) == 2, "16-bit types");
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(4 * TILE <= 160 * 1024, "two K and two V buffers must fit in LDS");
};

__device__ __forceinline__ int k_swz(int r) { return r & 15; }
// V: bits 0, 1, 2 of the row go to chunk bits 3, 2, 1.  The LDS serves a
// transposing read 32 lanes at a time; lanes 0-31 read 4 consecutive rows,
// each at two adjacent 32-byte chunk pairs.  Under this map those 8
// (row, pair) combinations fall in 8 distinct 32-byte bank groups, so the
// read is conflict-free (the previous map, 2 (r & 7), sent them to 4).
__device__ __forceinline__ int v_swz(int r) { return ((r & 1) << 3) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T, int BC, int MASK, int NW, int MINB>
__global__ __launch_bounds__(64 * NW, MINB) void fa_fwd_dma_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, MaskArgs mask,
    RowLayout lq, RowLayout lk, RowLayout lv, RowLayout lo,
    int H, int Nq, int Nk, int nqt, float c_log2) {
  using C = DmaCfg<T, BC, NW>;
  constexpr int D = C::D;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];   // K0 K1 V0 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int b = bh / H, h = bh - b * H;
  // Row pitches in bytes (D contiguous; validated to fit the 32-bit ranges).
  const uint32_t qs = (uint32_t)(lq.sn * 2), ks = (uint32_t)(lk.sn * 2), vs = (uint32_t)(lv.sn * 2);

  int n_eff = Nk;
  if constexpr (MASK == kMaskLen) {
    const int L = reinterpret_cast<const int*>(mask.ptr)[b];
    n_eff = L < 0 ? 0 : (L > Nk ? Nk : L);
  }
  const int ntiles = (n_eff + BC - 1) / BC;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + b * lq.sb + h * lq.sh, (uint32_t)Nq * qs);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + b * lk.sb + h * lk.sh, (uint32_t)n_eff * ks);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + b * lv.sb + h * lv.sh, (uint32_t)n_eff * vs);

  const int q_row = qt * C::BR + wave * 32 + ln;
  const bool q_ok = q_row < Nq;
  u32x4 qreg[C::QKS];
#pragma unroll
  for (int s = 0; s < C::QKS; ++s)
    qreg[s] = buf_load16(qr, (uint32_t)q_row * qs + (2 * s + lh) * 16);

  // Rows the DMA never reaches (past n_eff) must hold finite values: clear
  // both V buffers once.
  for (int i = tid; i < 2 * C::TILE / 16; i += C::NT)
    *reinterpret_cast<u32x4*>(smem + 2 * C::TILE + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // DMA of tile j into buffer j & 1.  Instruction i of this wave fills LDS
  // kilobyte (wave * DMA_PER_WAVE + i): rows 4 per kilobyte, this lane's
  // 16 bytes at row r, physical chunk lane % 16.
  auto dma_tile = [&](int j) {
    const uint32_t row0 = (uint32_t)(j * BC);
    uint8_t* kb = smem + (j & 1) * C::TILE;
    uint8_t* vb = smem + 2 * C::TILE + (j & 1) * C::TILE;
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
      const int kb_idx = wave * C::DMA_PER_WAVE + i;
      const int r = kb_idx * 4 + (lane >> 4);
      const int pc = lane & 15;
      const uint32_t koff = (row0 + r) * ks + ((pc ^ k_swz(r)) << 4);
      const uint32_t voff = (row0 + r) * vs + ((pc ^ v_swz(r)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kb + kb_idx * 1024), 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vb + kb_idx * 1024), 16, voff, 0, 0, 0);
    }
  };
  // Wait for this wave's DMA, then for everyone's.
  auto dma_wait_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };

  constexpr float kLazy = 8.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc[C::PVB];
#pragma unroll
  for (int p = 0; p < C::PVB; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;

  constexpr bool kPre = (MASK == kMaskAdd);
  const float cs = kPre ? 1.f : c_log2;
  // additive mask: this lane's query row (row 0 stands in for rows past Nq,
  // whose results are not stored)
  const float* mrow = nullptr;
  bool mvec = false;
  if constexpr (kPre) {
    mrow = reinterpret_cast<const float*>(mask.ptr) + b * mask.sb + h * mask.sh +
           (int64_t)(q_ok ? q_row : 0) * mask.sq;
    mvec = mask_rows_vec4(mask);
  }

  auto step = [&](int j, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint8_t* kb = smem + (j & 1) * C::TILE;
    const uint8_t* vb = smem + 2 * C::TILE + (j & 1) * C::TILE;
    dma_tile(j + 1);                      // past the last tile: reads zeros, never used
    const int kv0 = j * BC;

    // S^T = K Q^T; K operand reads of block G + 1 ride ahead of block G's MFMAs
    f32x16 s[C::SB];
    u32x4 ka[C::QKS];
    auto kread = [&](int G, int st) {
      const int r = 32 * G + ln;
      return *reinterpret_cast<const u32x4*>(kb + r * C::ROW + (((2 * st + lh) ^ k_swz(r)) << 4));
    };
#pragma unroll
    for (int st = 0; st < C::QKS; ++st) ka[st] = kread(0, st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int G = 0; G < C::SB; ++G) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[G][i] = 0.f;
#pragma unroll
      for (int st = 0; st < C::QKS; ++st) {
        const u32x4 a = ka[st];
        if (G + 1 < C::SB) ka[st] = kread(G + 1, st);
        s[G] = mfma_chunk<T>(a, qreg[st], s[G]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (MASKED) {
      if constexpr (kPre) {
        // additive mask, 4 consecutive keys per load (keys past Nk read -inf),
        // each quad loaded next to its use (the tile's scores hold the
        // registers); a whole tile of a key-contiguous aligned row takes
        // 16-byte loads
        auto add_mask = [&](auto vec_tag) {
          constexpr bool VEC = decltype(vec_tag)::value;
#pragma unroll
          for (int G = 0; G < C::SB; ++G)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 mq = mask_quad<VEC>(mrow, mask.sk, kv0 + 32 * G + 8 * g + 4 * lh, Nk);
#pragma unroll
              for (int r = 0; r < 4; ++r) s[G][4 * g + r] = __builtin_fmaf(s[G][4 * g + r], c_log2, mq[r] * kLog2e);
            }
        };
        if (mvec && kv0 + BC <= Nk) add_mask(BoolTag<true>{});
        else add_mask(BoolTag<false>{});
      } else {
#pragma unroll
        for (int G = 0; G < C::SB; ++G)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * G + 8 * (i >> 2) + 4 * lh + (i & 3);
            s[G][i] = key < n_eff ? s[G][i] : -INFINITY;
          }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int G = 0; G < C::SB; ++G)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[G][i]);
    mx = wave_max_halves(mx) * cs;
    if (__ballot(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int p = 0; p < C::PVB; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[p][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;

    float psum = -0.f;                            // -0 + x == x: the first add folds away
#pragma unroll
    for (int G = 0; G < C::SB; ++G)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[G][i], cs, -m_use));
        s[G][i] = p;
        psum += p;
      }
    l_run += psum;

    // O^T += V^T P^T.  Transposing reads: this lane, as source lane
    // 4k + t of its 16-lane group, fetches channels 4t..4t+3 of key k.
    const int gk = (lane & 15) >> 2, gt = lane & 3, ga = (lane >> 4) & 1;
#pragma unroll
    for (int G = 0; G < C::SB; ++G) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[G][cc * 8 + e];
        const u32x4 bop = pack_chunk<T>(pv);
#pragma unroll
        for (int p = 0; p < C::PVB; ++p) {
          const int lc = 4 * p + 2 * ga + (gt >> 1);        // logical 16-byte chunk of channel 32p + 16a + 4t
          const int r0 = 32 * G + 16 * cc + 4 * lh + gk;      // keys +0..3, then +8..11
          const int r1 = r0 + 8;
          const uint8_t* a0 = vb + r0 * C::ROW + ((lc ^ v_swz(r0)) << 4) + ((gt & 1) << 3);
          const uint8_t* a1 = vb + r1 * C::ROW + ((lc ^ v_swz(r1)) << 4) + ((gt & 1) << 3);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
          u32x4 a;
          a.x = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
          a.y = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
          a.z = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
          a.w = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
          acc[p] = mfma_chunk<T>(a, bop, acc[p]);
        }
      }
    }
    dma_wait_barrier();
  };

  dma_tile(0);
  dma_wait_barrier();
  if constexpr (kPre) {
    for (int j = 0; j < ntiles; ++j) step(j, BoolTag<true>{});
  } else {
    const int nfull = n_eff / BC;
    for (int j = 0; j < nfull; ++j) step(j, BoolTag<false>{});
    if (nfull < ntiles) step(nfull, BoolTag<true>{});
  }

  const float l_tot = wave_sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = O + b * lo.sb + h * lo.sh + (int64_t)q_row * lo.sn;
#pragma unroll
    for (int p = 0; p < C::PVB; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * p + 8 * g + 4 * lh;
        store4<T>(orow + d0, acc[p][4 * g] * inv, acc[p][4 * g + 1] * inv,
                  acc[p][4 * g + 2] * inv, acc[p][4 * g + 3] * inv);
      }
    if (LSE != nullptr && lh == 0)
      LSE[(size_t)bh * Nq + q_row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace fa
