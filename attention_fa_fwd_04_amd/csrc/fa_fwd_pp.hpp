// Attention forward for 16-bit types with D = 128 (no additive mask): the
// LDS-DMA staged kernel of fa_fwd_dma.hpp, rescheduled so that the two waves
// sharing a SIMD alternate between the matrix core and the vector ALU.
//
// Method: handbook page "算子加速：注意力、编译与融合", section
// "注意力：从 O(N²) 显存到分块" (running row max and denominator, rescaled
// accumulator, only O written).  Each wave owns 32 query rows, computes
// S^T = K Q^T with 32x32 MFMAs so a lane owns one query, and accumulates
// O^T += V^T P^T; 64-key tiles reach LDS by buffer-load DMA with the chunk
// swizzles of fa_fwd_dma.hpp.
//
// Schedule.  A workgroup has 8 waves; the hardware places waves w and w + 4
// on the same SIMD, so waves 0-3 form group A and waves 4-7 group B, one of
// each per SIMD.  The work of key tile t is split into two phases:
//   MFMA phase     P V of tile t-1, then S = K Q^T of tile t   (matrix core)
//   softmax phase  row max, exp2, row sum, narrowing of P      (vector ALU)
// Group A runs MFMA(0), softmax(0), MFMA(1), ...; group B runs the same
// sequence one phase later.  A workgroup barrier closes every phase, so in
// each phase one wave of every SIMD feeds the matrix core while the other
// runs the softmax; two barriers per tile.  Each phase pins its results
// before its closing barrier (the compiler would otherwise move softmax
// arithmetic past the barrier into the MFMA phase and undo the alternation).
//
// Operands.  In an MFMA phase the K operands of Q K^T are read from LDS
// during the P V steps (twelve of sixteen; the last four just before the
// MFMAs that use them) and the V operands one step ahead of their MFMAs.
//
// Tile traffic.  Two K and two V buffers; group A loads K tiles and group B
// V tiles, each wave a quarter, at the start of its softmax phase (which
// reads no LDS), from per-lane offsets computed once.  Group A loads K(t+1)
// in phase 2t + 1 (first read in phase 2t + 2; it replaces K(t-1), last read
// in phase 2t - 1) and waits for it before that phase's closing barrier.
// Group B loads V(t+1) in phase 2t + 2 (first read in phase 2t + 4; it
// replaces V(t-1), last read in phase 2t + 1) and waits for it before the
// closing barrier of phase 2t + 3; the transposing V reads of its MFMA phase
// in between make the compiler wait for it there already, about a phase
// after the issue.  A prologue loads K(0) with all eight waves; group B loads
// V(0) in phase 0.
//
// The ragged last tile (keys [nfull BC, n_eff)) is processed first with all
// eight waves in step, so the phase loop sees only full tiles.
//
// The row max needs both lane halves (keys of one query are split across
// them).  With the lazy rescale the hot path only compares each half's max
// with the shared running max; the halves are combined only when some row
// crosses the threshold, and once at the end for the denominator.
#pragma once

#include "fa_common.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_fwd_dma.hpp"

#include <type_traits>

namespace fa {

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// An opaque copy: values derived from it are recomputed where they are used
// instead of being hoisted out of the tile loop and held in registers.
__device__ __forceinline__ uint32_t launder(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// Workgroup barrier that orders LDS accesses (compiler and hardware) but,
// unlike __syncthreads(), does not wait for outstanding DMA.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int BC, int MASK>
__global__ __launch_bounds__(512, 1) void fa_fwd_pp_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, MaskArgs mask,
    RowLayout lq, RowLayout lk, RowLayout lv, RowLayout lo,
    int H, int Nq, int Nk, int nqt, float c_log2) {
  constexpr int NW = 8;
  using C = DmaCfg<T, BC, NW>;
  constexpr int D = C::D, SB = C::SB, QKS = C::QKS, PVB = C::PVB;
  constexpr int KB_PER_TILE = C::TILE / 1024;          // 1 KB DMA instructions per tile
  constexpr int KB_ALL = KB_PER_TILE / NW;             // per wave when all 8 load
  constexpr int KB_B = KB_PER_TILE / 4;                // per wave when one group of four loads
  static_assert(KB_PER_TILE % NW == 0, "tile must split over 8 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];   // K0 K1 V0 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int ln = lane & 31, lh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int b = bh / H, h = bh - b * H;
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
  u32x4 qreg[QKS];
#pragma unroll
  for (int s = 0; s < QKS; ++s)
    qreg[s] = buf_load16(qr, (uint32_t)q_row * qs + (2 * s + lh) * 16);

  for (int i = tid; i < 2 * C::TILE / 16; i += C::NT)
    *reinterpret_cast<u32x4*>(smem + 2 * C::TILE + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // DMA of kilobytes [kb0, kb0 + n) of tile j (4 rows per kilobyte) into buf;
  // the lane landing at physical chunk lane % 16 of row r fetches logical
  // chunk (lane % 16) ^ swz(r).  The whole offset is in the range-checked
  // vector offset, so rows past n_eff read as zero.
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* buf, int j, int kb0, int n, bool is_v) {
    const uint32_t l = launder((uint32_t)lane);
    const uint32_t pitch = is_v ? vs : ks;
    for (int i = 0; i < n; ++i) {
      const int kb_idx = kb0 + i;
      const int r = kb_idx * 4 + (int)(l >> 4);
      const int lc = (int)(l & 15) ^ (is_v ? v_swz(r) : k_swz(r));
      const uint32_t off = (uint32_t)(j * BC + r) * pitch + (uint32_t)(lc << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + kb_idx * 1024), 16, off, 0, 0, 0);
    }
  };
  uint8_t* const kbuf0 = smem;
  uint8_t* const vbuf0 = smem + 2 * C::TILE;

  constexpr float kLazy = 8.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc[PVB];
#pragma unroll
  for (int p = 0; p < PVB; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;
  f32x16 s[SB];
  u32x4 pb[SB][2];   // P^T operand of the pending P V, 8 keys per chunk

  static_assert(MASK != kMaskAdd, "additive masks use fa_fwd_dma_kernel");
  const float cs = c_log2;

  // Lane-constant parts of the operand addresses, computed once.
  // K: row (lane % 32) of each 32-key block, chunk (2 st + lh) ^ k_swz(r)
  //    = 2 st ^ ky.
  const uint32_t k_lane = (uint32_t)(lane & 31) * C::ROW;
  const int ky = (lane >> 5) ^ (lane & 15);
  // V (transposing reads): this lane, as source lane 4k + t of its 16-lane
  // group, fetches channels 4t..4t+3 of key k (keys +0..3, then +8..11).
  // Row r = 32 G + 16 cc + 4 lh + gk (+ 8) has swizzle v_swz(4 lh + gk): G,
  // cc and the +8 only add constant row offsets.
  uint32_t vaddr[PVB];
  {
    const int gk = (lane & 15) >> 2, gt = lane & 3, ga = (lane >> 4) & 1;
    const int r_l = 4 * (lane >> 5) + gk;
    const uint32_t vbase = r_l * C::ROW + ((gt & 1) << 3);
#pragma unroll
    for (int p = 0; p < PVB; ++p) vaddr[p] = vbase + (((4 * p + 2 * ga + (gt >> 1)) ^ v_swz(r_l)) << 4);
  }

  // ---- MFMA phase: O^T += V^T P^T for the previous tile, then S^T = K Q^T
  // for this one.  P V runs first so the narrowed P is dead before S is
  // produced; twelve of the sixteen K operands of Q K^T are read during the
  // P V steps, the V operands one step ahead of their MFMAs.
  auto mma_phase = [&](const uint8_t* kb, const uint8_t* vb, auto do_pv, auto do_qk) {
    constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
    constexpr int KCH = SB * QKS;                     // K operand chunks per tile
    u32x4 ka[KCH];
    auto kread = [&](int c) {                         // chunk c = st * SB + G
      const int st = c / SB, G = c % SB;
      ka[c] = *reinterpret_cast<const u32x4*>(kb + k_lane + 32 * G * C::ROW + (((2 * st) ^ ky) << 4));
    };
    if constexpr (PV) {
      u32x4 va[2][PVB];
      auto vread = [&](auto kk) {
        constexpr int k = decltype(kk)::value;
        constexpr int off = (32 * (k >> 1) + 16 * (k & 1)) * C::ROW;
        static_for<PVB>([&](auto pp) {
          constexpr int p = decltype(pp)::value;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + vaddr[p] + off));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + vaddr[p] + off + 8 * C::ROW));
          va[k % 2][p].x = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
          va[k % 2][p].y = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
          va[k % 2][p].z = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
          va[k % 2][p].w = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
        });
      };
      constexpr int KSTEPS = 2 * SB;
      constexpr int KPER = (KCH - 4) / KSTEPS;         // K chunks read per P V step
      vread(std::integral_constant<int, 0>{});
      static_for<KSTEPS>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k + 1 < KSTEPS) vread(std::integral_constant<int, k + 1>{});
        if constexpr (QK) {
#pragma unroll
          for (int c = k * KPER; c < (k + 1) * KPER; ++c) kread(c);
        }
#pragma unroll
        for (int p = 0; p < PVB; ++p) acc[p] = mfma_chunk<T>(va[k % 2][p], pb[k >> 1][k & 1], acc[p]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (QK) {
#pragma unroll
      for (int c = 0; c < KCH - 4; ++c) kread(c);
    }
    if constexpr (QK) {
#pragma unroll
      for (int c = KCH - 4; c < KCH; ++c) kread(c);   // used by the last four MFMAs
#pragma unroll
      for (int G = 0; G < SB; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[G][i] = 0.f;
#pragma unroll
      for (int st = 0; st < QKS; ++st)
#pragma unroll
        for (int G = 0; G < SB; ++G) s[G] = mfma_chunk<T>(ka[st * SB + G], qreg[st], s[G]);
    }
  };

  // ---- softmax phase for tile t: S -> P (narrowed into pb), m, l, rescale
  auto softmax_phase = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kv0 = t * BC;
    if constexpr (MASKED) {
      // Keys at or past n_eff (only in the last tile) drop out: compare the
      // key's offset within the tile with one per-lane limit.
      const int lim = (int)launder((uint32_t)(n_eff - kv0 - 4 * lh));
#pragma unroll
      for (int G = 0; G < SB; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * G + 8 * (i >> 2) + (i & 3) >= lim) s[G][i] = -INFINITY;
    }
    float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int G = 0; G < SB; ++G)
#pragma unroll
      for (int i = 0; i < 16; ++i) mq[i & 3] = fmaxf(mq[i & 3], s[G][i]);
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx *= cs;                                   // this half's keys only
    if (__ballot(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, wave_max_halves(mx));
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int p = 0; p < PVB; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[p][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int G = 0; G < SB; ++G)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[G][cc * 8 + e], cs, -m_use));
          psum += pv[e];
        }
        pb[G][cc] = pack_chunk<T>(pv);
      }
    l_run += psum;
    // the phase's results exist before its closing barrier (the compiler
    // would otherwise sink this arithmetic into the next phase)
    asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(l_run), "v"(m_run));
  };

  // The ragged last tile (keys [nfull BC, n_eff)) goes first, outside the
  // phase loop, with all eight waves in step; the loop then only sees full
  // tiles.  The order of key tiles does not change the result beyond rounding.
  const int nfull = n_eff / BC;
  if (nfull < ntiles) {
    dma(kr, kbuf0, nfull, wave * KB_ALL, KB_ALL, false);
    dma(vr, vbuf0, nfull, wave * KB_ALL, KB_ALL, true);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    mma_phase(kbuf0, vbuf0, BoolTag<false>{}, BoolTag<true>{});
    softmax_phase(nfull, BoolTag<true>{});
    mma_phase(kbuf0, vbuf0, BoolTag<true>{}, BoolTag<false>{});
    __syncthreads();
  }

  const int nt = nfull;
  // Prologue: all eight waves load K(0).
  if (nt > 0) dma(kr, kbuf0, 0, wave * KB_ALL, KB_ALL, false);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();

  // Phase loop, one straight-line schedule per group (2 nt + 2 barriers
  // each).  Tile t: K(t) in K buffer t & 1, V(t) in V buffer t & 1.
  auto kbuf = [&](int t) { return kbuf0 + (t & 1) * C::TILE; };
  auto vbuf = [&](int t) { return vbuf0 + (t & 1) * C::TILE; };
  if (nt > 0) {
    // Tile DMA: group A loads K tiles, group B loads V tiles, each wave a
    // quarter, from per-lane offsets computed once (tile j adds j * BC rows).
    const int kb4 = (wave & 3) * KB_B;
    uint32_t offs[KB_B];
    {
      const uint32_t pitch = grp == 0 ? ks : vs;
#pragma unroll
      for (int i = 0; i < KB_B; ++i) {
        const int r = (kb4 + i) * 4 + (lane >> 4);
        const int sw = grp == 0 ? k_swz(r) : v_swz(r);
        offs[i] = (uint32_t)r * pitch + (uint32_t)(((lane & 15) ^ sw) << 4);
      }
    }
    auto dma4 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* buf, int j, uint32_t pitch, const uint32_t* o) {
      const uint32_t row_off = (uint32_t)(j * BC) * pitch;
#pragma unroll
      for (int i = 0; i < KB_B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (kb4 + i) * 1024), 16, o[i] + row_off, 0, 0, 0);
    };
    if (grp == 0) {
      mma_phase(kbuf(0), vbuf(0), BoolTag<false>{}, BoolTag<true>{});
      lds_barrier();                                            // phase 0
      for (int t = 0; t + 1 < nt; ++t) {
        // phase 2t + 1: K(t + 1), first read in phase 2t + 2, replaces K(t - 1),
        // last read in phase 2t - 1
        dma4(kr, kbuf(t + 1), t + 1, ks, offs);
        softmax_phase(t, BoolTag<false>{});
        __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
        lds_barrier();                                          // phase 2t + 1
        mma_phase(kbuf(t + 1), vbuf(t), BoolTag<true>{}, BoolTag<true>{});
        lds_barrier();                                          // phase 2t + 2
      }
      softmax_phase(nt - 1, BoolTag<false>{});
      lds_barrier();                                            // phase 2nt - 1
      mma_phase(kbuf(0), vbuf(nt - 1), BoolTag<true>{}, BoolTag<false>{});
      lds_barrier();                                            // phase 2nt
      lds_barrier();                                            // phase 2nt + 1
    } else {
      dma4(vr, vbuf(0), 0, vs, offs);                           // V(0), buffer unused yet
      lds_barrier();                                            // phase 0
      mma_phase(kbuf(0), vbuf(0), BoolTag<false>{}, BoolTag<true>{});
      __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0): V(0) landed
      lds_barrier();                                            // phase 1
      for (int t = 0; t + 1 < nt; ++t) {
        // phase 2t + 2: V(t + 1), first read in phase 2t + 4, replaces V(t - 1),
        // last read in phase 2t + 1
        dma4(vr, vbuf(t + 1), t + 1, vs, offs);
        softmax_phase(t, BoolTag<false>{});
        lds_barrier();                                          // phase 2t + 2
        mma_phase(kbuf(t + 1), vbuf(t), BoolTag<true>{}, BoolTag<true>{});
        __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0): V(t + 1) landed
        lds_barrier();                                          // phase 2t + 3
      }
      softmax_phase(nt - 1, BoolTag<false>{});
      lds_barrier();                                            // phase 2nt
      mma_phase(kbuf(0), vbuf(nt - 1), BoolTag<true>{}, BoolTag<false>{});
      lds_barrier();                                            // phase 2nt + 1
    }
  }

  const float l_tot = wave_sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = O + b * lo.sb + h * lo.sh + (int64_t)q_row * lo.sn;
#pragma unroll
    for (int p = 0; p < PVB; ++p)
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
