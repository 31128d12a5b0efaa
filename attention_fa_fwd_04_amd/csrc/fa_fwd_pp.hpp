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
// Group B loads V(t+1) in phase 2t + 2 (it replaces V(t-1), last read in
// phase 2t + 1) and waits for it before that phase's closing barrier too.
// Each group reads the first P V step's V operands at the end of its softmax
// phase, where its wave would otherwise idle at the barrier: group A reads
// V(t) in phase 2t + 1, group B in phase 2t + 2, both after V(t) landed (end
// of phase 2t).  A prologue loads K(0) with all eight waves; group B loads
// V(0) in phase 0 and waits for it before phase 0 ends, since group A reads
// it at the end of phase 1.
//
// The ragged last tile (keys [nfull BC, n_eff)) is processed first with all
// eight waves in step, so the phase loop sees only full tiles.
//
// The row max needs both lane halves (keys of one query are split across
// them).  With the lazy rescale the hot path only compares each half's max
// with the shared running max; the halves are combined only when some row
// crosses the threshold, and once at the end for the denominator.
//
// Even split of the key tiles (SPLIT = true, no mask).  When the number of
// query blocks is not close to a multiple of the CU count, the last round
// of workgroups leaves CUs idle (432 blocks of 256 rows on 256 CUs run in
// two rounds, the second 69 % full).  The split launch runs one workgroup
// per CU and hands each the same number of (query block, key tile) units in
// block-major order, so a workgroup finishes the key tiles of a block its
// predecessor started, takes whole blocks, and starts a block its successor
// finishes.  A block split between two workgroups is the same online
// softmax over two disjoint key ranges: the part that arrives first (an
// arrival counter per split) leaves its unnormalised accumulator, running
// max and denominator in the workspace, and the part that arrives second
// combines the two by the handbook's rescale, exp(m_part - m), and stores O
// and lse.  A part writes its partial unless it finds the other counted
// already; both write only if they arrive together.  The
// combination is written as a function of (first-range part, second-range
// part) whichever arrives last, so the result does not depend on arrival
// order.  Both split parts of a workgroup run before its whole blocks, so
// the combining traffic overlaps other workgroups' compute.
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
// Workspace of the split launch.  cnt[s] counts the parts of split s that
// have arrived; it returns to zero when the second one arrives, so a
// workspace that starts zeroed stays zeroed between calls.
struct SplitArgs {
  unsigned* cnt;    // [grid + 1]
  float* part;      // [grid + 1][2][kPartFloats]
  int64_t units;    // query blocks x key tiles per block
  int tiles;        // key tiles per query block
};
// One part: 8 waves x 16 four-float accumulator chunks x 64 lanes, then
// (running max, denominator) per lane.
constexpr int kPartAccFloats = 8 * 16 * 64 * 4;
constexpr int kPartFloats = kPartAccFloats + 8 * 64 * 2;
// Segments of one workgroup of the split launch: at most two split parts
// plus the whole blocks of its range (the host keeps this bound).
constexpr int kMaxSegments = 16;

// Workgroup barrier that orders LDS accesses (compiler and hardware) but,
// unlike __syncthreads(), does not wait for outstanding DMA.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The two-group phase schedule over nt full key tiles, shared by the D = 128
// phase-alternating kernels (the schedule and buffer lifetimes are those of
// the header above).  Tile t lives in K buffer t & 1 and V buffer t & 1.
//   mma(tk, tv, pv, qk, pre)  MFMA phase on K tile tk and V tile tv; the
//                             BoolTag flags select P V of the previous tile,
//                             Q K^T of tile tk, and V operands of the first
//                             P V step already read
//   softmax(t)                softmax phase of tile t
//   load_k(t), load_v(t)      this wave's share of tile t's DMA (group A
//                             loads K tiles, group B V tiles)
//   vread_first(t)            the first P V step's V operands of tile t
// K(0) must be resident on entry; every wave passes 2 nt + 2 barriers.
template <typename Mma, typename Soft, typename LoadK, typename LoadV, typename VFirst>
__device__ __forceinline__ void pp_phase_loop(int grp, int nt, Mma&& mma, Soft&& softmax, LoadK&& load_k,
                                              LoadV&& load_v, VFirst&& vread_first) {
  if (grp == 0) {
    mma(0, 0, BoolTag<false>{}, BoolTag<true>{}, BoolTag<false>{});
    lds_barrier();                                            // phase 0
    for (int t = 0; t + 1 < nt; ++t) {
      // phase 2t + 1: K(t + 1), first read in phase 2t + 2, replaces K(t - 1),
      // last read in phase 2t - 1
      load_k(t + 1);
      softmax(t);
      __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
      vread_first(t);                                         // V(t): landed by the end of phase 2t
      lds_barrier();                                          // phase 2t + 1
      mma(t + 1, t, BoolTag<true>{}, BoolTag<true>{}, BoolTag<true>{});
      lds_barrier();                                          // phase 2t + 2
    }
    softmax(nt - 1);
    vread_first(nt - 1);
    lds_barrier();                                            // phase 2nt - 1
    mma(0, nt - 1, BoolTag<true>{}, BoolTag<false>{}, BoolTag<true>{});
    lds_barrier();                                            // phase 2nt
    lds_barrier();                                            // phase 2nt + 1
  } else {
    load_v(0);                                                // V(0), buffer unused yet
    // V(0) must be resident by the end of phase 0: group A reads it at the
    // end of its first softmax phase, phase 1
    __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0): V(0) landed
    lds_barrier();                                            // phase 0
    mma(0, 0, BoolTag<false>{}, BoolTag<true>{}, BoolTag<false>{});
    lds_barrier();                                            // phase 1
    for (int t = 0; t + 1 < nt; ++t) {
      // phase 2t + 2: V(t + 1), first read at the end of phase 2t + 3,
      // replaces V(t - 1), last read in phase 2t + 1
      load_v(t + 1);
      softmax(t);
      __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0): V(t + 1) landed
      vread_first(t);
      lds_barrier();                                          // phase 2t + 2
      mma(t + 1, t, BoolTag<true>{}, BoolTag<true>{}, BoolTag<true>{});
      lds_barrier();                                          // phase 2t + 3
    }
    softmax(nt - 1);
    vread_first(nt - 1);
    lds_barrier();                                            // phase 2nt
    mma(0, nt - 1, BoolTag<true>{}, BoolTag<false>{}, BoolTag<true>{});
    lds_barrier();                                            // phase 2nt + 1
  }
}

template <typename T, int BC, int MASK, bool SPLIT>
__global__ __launch_bounds__(512, 1) void fa_fwd_pp_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, MaskArgs mask,
    RowLayout lq, RowLayout lk, RowLayout lv, RowLayout lo,
    int H, int Nq, int Nk, int nqt, float c_log2, SplitArgs sk) {
  constexpr int NW = 8;
  using C = DmaCfg<T, BC, NW>;
  constexpr int D = C::D, SB = C::SB, QKS = C::QKS, PVB = C::PVB;
  constexpr int KB_PER_TILE = C::TILE / 1024;          // 1 KB DMA instructions per tile
  constexpr int KB_ALL = KB_PER_TILE / NW;             // per wave when all 8 load
  constexpr int KB_B = KB_PER_TILE / 4;                // per wave when one group of four loads
  static_assert(KB_PER_TILE % NW == 0, "tile must split over 8 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];   // K0 K1 V0 V1
  __shared__ unsigned arrival;
  static_assert(!SPLIT || MASK == kMaskNone, "the split launch takes no mask");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int ln = lane & 31, lh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // The split launch takes contiguous [B, H, N, 128] tensors only, so its
  // row pitches are constants (fewer scalar registers live across segments).
  const uint32_t qs = SPLIT ? 2u * D : (uint32_t)(lq.sn * 2);
  const uint32_t ks = SPLIT ? 2u * D : (uint32_t)(lk.sn * 2);
  const uint32_t vs = SPLIT ? 2u * D : (uint32_t)(lv.sn * 2);

  // Segments: (query block, key tiles [t0, t1)).  Without the split, one
  // segment: the whole key range of block `logical`.  With it, units
  // [u0, u1) of the block-major (block, tile) order: the first part of the
  // block containing u1 (if u1 falls inside one), the second part of the
  // block containing u0 (if u0 falls inside one), then the whole blocks.
  // The split launch lists its segments in LDS once (job, t0, t1, part,
  // slot), so nothing but the segment index stays live across them.
  __shared__ int segd[kMaxSegments][5];
  __shared__ int nseg_s;
  if constexpr (SPLIT) {
    if (tid == 0) {
      const int64_t G = gridDim.x, TT = sk.tiles;
      const int64_t u0 = (int64_t)logical * sk.units / G;
      const int64_t u1 = ((int64_t)logical + 1) * sk.units / G;
      int n = 0;
      auto put = [&](int64_t job, int64_t t0, int64_t t1, int part, int slot) {
        if (n < kMaxSegments) {
          segd[n][0] = (int)job; segd[n][1] = (int)t0; segd[n][2] = (int)t1; segd[n][3] = part; segd[n][4] = slot;
        }
        ++n;
      };
      if (u1 % TT != 0) put(u1 / TT, 0, u1 % TT, 0, logical + 1);
      if (u0 % TT != 0) put(u0 / TT, u0 % TT, TT, 1, logical);
      for (int64_t j = (u0 + TT - 1) / TT; j < u1 / TT; ++j) put(j, 0, TT, -1, 0);
      nseg_s = n < kMaxSegments ? n : kMaxSegments;
    }
    __syncthreads();
  }
  // One segment: query block `job`, key tiles [t0, t1) (t1 ignored without
  // the split); part 0 / 1 is the first / second key range of split `slot`,
  // -1 a whole block.
  auto segment = [&](const int job, const int t0, const int t1, const int part, const int slot) {
  const int bh = job / nqt, qt = job - bh * nqt;
  const int b = bh / H, h = bh - b * H;

  int n_all = Nk;
  if constexpr (MASK == kMaskLen) {
    const int L = reinterpret_cast<const int*>(mask.ptr)[b];
    n_all = L < 0 ? 0 : (L > Nk ? Nk : L);
  }
  // keys [k0, k0 + n_eff) of this segment; the K and V ranges start at k0
  int k0 = 0, n_eff = n_all;
  if constexpr (SPLIT) {
    k0 = t0 * BC;
    n_eff = (t1 >= sk.tiles ? n_all : t1 * BC) - k0;
  }
  const int ntiles = (n_eff + BC - 1) / BC;
  const T* qh = Q + b * lq.sb + h * lq.sh;
  const T* kh = K + b * lk.sb + h * lk.sh;
  const T* vh = V + b * lv.sb + h * lv.sh;
  T* oh = O + b * lo.sb + h * lo.sh;
  if constexpr (SPLIT) {
    const int64_t ho = (int64_t)bh * Nq * D;
    qh = Q + ho;
    kh = K + ho + (int64_t)k0 * D;
    vh = V + ho + (int64_t)k0 * D;
    oh = O + ho;
  }
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, (uint32_t)Nq * qs);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh, (uint32_t)n_eff * ks);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vh, (uint32_t)n_eff * vs);

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

  // V operands of the pending P V: step k (16 keys) in va[k % 2].
  u32x4 va[2][PVB];
  auto vread = [&](const uint8_t* vb, auto kk) {
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
  // The first step's V operands of a phase loop's P V are read at the end of
  // the preceding softmax phase, whose wave otherwise idles at the barrier:
  // the V tile is resident by then and no DMA writes that buffer until after
  // the MFMA phase that uses it.
  auto vread_first = [&](const uint8_t* vb) { vread(vb, std::integral_constant<int, 0>{}); };

  // ---- MFMA phase: O^T += V^T P^T for the previous tile, then S^T = K Q^T
  // for this one.  P V runs first so the narrowed P is dead before S is
  // produced; twelve of the sixteen K operands of Q K^T are read during the
  // P V steps, the V operands one step ahead of their MFMAs (the first step's
  // already in va[0] when PRE).
  auto mma_phase = [&](const uint8_t* kb, const uint8_t* vb, auto do_pv, auto do_qk, auto pre_tag) {
    constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
    constexpr bool PRE = decltype(pre_tag)::value;
    constexpr int KCH = SB * QKS;                     // K operand chunks per tile
    u32x4 ka[KCH];
    auto kread = [&](int c) {                         // chunk c = st * SB + G
      const int st = c / SB, G = c % SB;
      ka[c] = *reinterpret_cast<const u32x4*>(kb + k_lane + 32 * G * C::ROW + (((2 * st) ^ ky) << 4));
    };
    if constexpr (PV) {
      constexpr int KSTEPS = 2 * SB;
      constexpr int KPER = (KCH - 4) / KSTEPS;         // K chunks read per P V step
      if constexpr (!PRE) vread(vb, std::integral_constant<int, 0>{});
      static_for<KSTEPS>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k + 1 < KSTEPS) vread(vb, std::integral_constant<int, k + 1>{});
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
    float psum = -0.f;                            // -0 + x == x: the first add folds away
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
  if (!SPLIT && nfull < ntiles) {             // the split launch needs N % BC == 0
    dma(kr, kbuf0, nfull, wave * KB_ALL, KB_ALL, false);
    dma(vr, vbuf0, nfull, wave * KB_ALL, KB_ALL, true);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    mma_phase(kbuf0, vbuf0, BoolTag<false>{}, BoolTag<true>{}, BoolTag<false>{});
    softmax_phase(nfull, BoolTag<true>{});
    mma_phase(kbuf0, vbuf0, BoolTag<true>{}, BoolTag<false>{}, BoolTag<false>{});
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
    pp_phase_loop(
        grp, nt,
        [&](int tk, int tv, auto pv, auto qk, auto pre) { mma_phase(kbuf(tk), vbuf(tv), pv, qk, pre); },
        [&](int t) { softmax_phase(t, BoolTag<false>{}); },
        [&](int t) { dma4(kr, kbuf(t), t, ks, offs); }, [&](int t) { dma4(vr, vbuf(t), t, vs, offs); },
        [&](int t) { vread_first(vbuf(t)); });
  }

  float l_tot = wave_sum_halves(l_run);
  float m_fin = m_run;
  if constexpr (SPLIT) {
    if (part >= 0) {
      // Leave this part, count it, and combine if the other part is in.
      // The two parts may run on different XCDs (separate L2s): partials
      // are written through and read back at device scope (the sc1 cache
      // policy) instead of fencing, which would write back and invalidate
      // the whole L2 and with it the K/V tiles other workgroups reuse.
      constexpr int kDeviceScope = 16;          // sc1
      const __amdgpu_buffer_rsrc_t pr =
          make_rsrc(sk.part, (uint32_t)((gridDim.x + 1) * 2 * (uint32_t)kPartFloats * 4u));
      const uint32_t mine = (uint32_t)(slot * 2 + part) * (uint32_t)kPartFloats * 4u;
      const uint32_t other = (uint32_t)(slot * 2 + (1 - part)) * (uint32_t)kPartFloats * 4u;
      const uint32_t lane_acc = (uint32_t)(wave * 16 * 64 + lane) * 16u;
      const uint32_t lane_ml = (uint32_t)kPartAccFloats * 4u + (uint32_t)(wave * 64 + lane) * 8u;
      // A part that finds the other already counted skips writing its own:
      // the counter reaches 1 only after that part's partial is written.
      if (tid == 0) arrival = __hip_atomic_load(sk.cnt + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (arrival == 0) {
#pragma unroll
        for (int p = 0; p < PVB; ++p)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = {acc[p][4 * g], acc[p][4 * g + 1], acc[p][4 * g + 2], acc[p][4 * g + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), pr,
                                                   (int)(mine + lane_acc + (4 * p + g) * 64 * 16), 0, kDeviceScope);
          }
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{m_run, l_tot}), pr,
                                              (int)(mine + lane_ml), 0, kDeviceScope);
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's part is written
      }
      __syncthreads();
      if (tid == 0) arrival = atomicInc(sk.cnt + slot, 1u);
      __syncthreads();
      if (arrival == 0) return;                 // first to arrive: the other part stores
      f32x4 po[PVB * 4];
#pragma unroll
      for (int c = 0; c < PVB * 4; ++c)
        po[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              pr, (int)(other + lane_acc + c * 64 * 16), 0, kDeviceScope));
      const f32x2 ml = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                    pr, (int)(other + lane_ml), 0, kDeviceScope));
      // (first-range part, second-range part) whichever this is
      const bool first = part == 0;
      const float ma = first ? m_run : ml.x, mb = first ? ml.x : m_run;
      const float la = first ? l_tot : ml.y, lb = first ? ml.y : l_tot;
      const float mm = fmaxf(ma, mb);
      const float ref = mm == -INFINITY ? 0.f : mm;
      const float wa = __builtin_amdgcn_exp2f(ma - ref), wb = __builtin_amdgcn_exp2f(mb - ref);
#pragma unroll
      for (int p = 0; p < PVB; ++p)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = po[4 * p + g];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float own = acc[p][4 * g + e];
            const float a = first ? own : x[e], bb = first ? x[e] : own;
            acc[p][4 * g + e] = a * wa + bb * wb;
          }
        }
      l_tot = la * wa + lb * wb;
      m_fin = mm;
    }
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = oh + (int64_t)q_row * (SPLIT ? D : lo.sn);
#pragma unroll
    for (int p = 0; p < PVB; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * p + 8 * g + 4 * lh;
        store4<T>(orow + d0, acc[p][4 * g] * inv, acc[p][4 * g + 1] * inv,
                  acc[p][4 * g + 2] * inv, acc[p][4 * g + 3] * inv);
      }
    if (LSE != nullptr && lh == 0)
      LSE[(size_t)bh * Nq + q_row] = l_tot > 0.f ? (m_fin + log2f(l_tot)) * kLn2 : -INFINITY;
  }
  };

  if constexpr (SPLIT) {
    const int nseg = __builtin_amdgcn_readfirstlane(nseg_s);
    for (int seg = 0; seg < nseg; ++seg)
      segment(__builtin_amdgcn_readfirstlane(segd[seg][0]), __builtin_amdgcn_readfirstlane(segd[seg][1]),
              __builtin_amdgcn_readfirstlane(segd[seg][2]), __builtin_amdgcn_readfirstlane(segd[seg][3]),
              __builtin_amdgcn_readfirstlane(segd[seg][4]));
  } else {
    segment(logical, 0, 0, -1, 0);
  }
}

}  // namespace fa
