// INT8-QK / 16-bit-PV attention main loop with the phase-alternating
// schedule of fa_fwd_pp.hpp (handbook page "算子加速：注意力、编译与融合",
// section "SageAttention": INT8 Q K^T on integer matrix cores, P V with
// 16-bit operands).
//
// Arithmetic: exact int32 scores S = Q8 K8^T, scaled by sq * sk * scale
// log2(e); exact running row max per 64-key tile (P <= 1 against it, no lazy
// rescale); P rounded to the input's 16-bit type for the P V MFMA; l sums the
// unrounded P; O = acc / l.  Tiles are visited in key order, the ragged last
// tile last, so every P is rounded against the running max of the tiles up
// to its own, the order the emulation fixes.
// A key-length mask shortens the key range.  A per-key row term is added to
// every scaled score, its values for a tile loaded while the tile's Q K^T
// runs: an additive mask times log2(e) (scale, then the mask), or with Q
// smoothing (SQ) the compensation row of the wave's 64-token query block,
// which the prepass tabulates in log2 units.
//
// Schedule.  8 waves of 32 query rows, one workgroup per CU; waves w and
// w + 4 share a SIMD, so waves 0-3 (group A) and 4-7 (group B) hold one wave
// per SIMD each.  Key tile t splits into
//   MFMA phase     P V of tile t-1 (sixteen 16-bit 32x32x16), then S = K Q^T
//                  of tile t (eight INT8 32x32x32)              (matrix core)
//   softmax phase  row max, rescale, exp2, row sum, narrowing of P (vector)
// with group B one phase behind group A and a workgroup barrier closing every
// phase.  The MFMA phase (768 matrix-core cycles) is the longer one, as in
// the bf16 kernel.
//
// Tiles.  An int8 K tile (64 rows x 128 bytes, 8 KB) and a 16-bit V^T tile
// from the prepass (128 channel rows x 64 keys, 128 bytes, 16 KB), both with
// the chunk swizzle (r / 2) % 8 of 128-byte rows: two of each, filled by
// buffer-load DMA.  V^T rows are read with ds_read_b128 (one 16-byte operand
// chunk per lane and MFMA), half the LDS instructions of transposing reads
// of V rows (the bf16 kernel's form, within 0.5 % of it in time here).
// Group A loads K(t+1) at the start of its
// softmax phase 2t + 1 (two 1 KB instructions per wave), group B loads
// V(t+1) at the start of its softmax phase 2t + 2 (four per wave); each
// waits for its own DMA before the phase's closing barrier; the schedule
// is fa_fwd_pp.hpp's pp_phase_loop, with the buffer lifetimes of
// fa_fwd_pp_kernel.  Each group reads the first P V step's V operands at the
// end of its softmax phase.
#pragma once

#include "fa_int8qk.hpp"
#include "fa_fwd_pp.hpp"

namespace fa {

template <typename T, int MASK, bool SQ>
__global__ __launch_bounds__(512, 1) void fa_int8qk_pv16_pp_kernel(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const T* __restrict__ vt,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ comp, MaskArgs mask,
    T* __restrict__ O, float* __restrict__ LSE, int H, int N, int npad, int groups, int nqt, float c_log2) {
  constexpr int D = 128, BC = kInt8Bc, BR = 256;
  constexpr int KBYTES = BC * D;                // int8 K tile, 128-byte rows
  constexpr int VROW = 2 * BC;                  // 16-bit V^T row (64 keys), 128 bytes
  constexpr int VBYTES = D * VROW;
  static_assert(KBYTES == 8192 && VBYTES == 16384, "8 and 16 DMA instructions per tile");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * KBYTES + 2 * VBYTES];   // K0 K1 V0 V1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
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
  const int nt = n_eff / BC;                    // full tiles: the phase loop

  const int8_t* Qh = q8 + (size_t)bh * npad * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k8 + (size_t)bh * npad * D, (uint32_t)npad * D);
  // V^T [D, npad] in the prepass's key order; keys past N are zero there
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vt + (size_t)bh * D * npad, (uint32_t)D * npad * 2);

  const int q_row = qt * BR + wave * 32 + ln;
  const bool q_ok = q_row < N;
  // rows past N are zero codes in the workspace; rows past npad repeat its last
  u32x4 qreg[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qreg[s] = *reinterpret_cast<const u32x4*>(Qh + (size_t)min(q_row, npad - 1) * D + (2 * s + lh) * 16);
  // every query of a wave lies in one 64-token scale block
  const float sq_w = sq[(size_t)bh * groups + min((qt * BR + wave * 32) / kQBlock, groups - 1)];
  const float* skh = sk + (size_t)bh * groups;
  // The per-key row term: an additive mask's row for this lane's query (row
  // 0 stands in for rows past N, whose results are not stored), or the
  // compensation row of the wave's query block (rows of npad floats,
  // 256-byte aligned); mk holds the current tile's values.
  constexpr bool kAdd = MASK == kMaskAdd;
  constexpr bool kRowTerm = kAdd || SQ;
  static_assert(!(SQ && kAdd), "Q smoothing takes no additive mask");
  const float* mrow = nullptr;
  int64_t mstride = 1;
  bool mvec = false;
  if constexpr (kAdd) {
    mrow = reinterpret_cast<const float*>(mask.ptr) + b * mask.sb + h * mask.sh + (int64_t)(q_ok ? q_row : 0) * mask.sq;
    mstride = mask.sk;
    mvec = mask_rows_vec4(mask);
  }
  if constexpr (SQ) {
    mrow = comp + ((size_t)bh * groups + min((qt * BR + wave * 32) / kQBlock, groups - 1)) * npad;
    mvec = true;
  }
  float mk[32];

  // DMA offsets (tile 0) of 1 KB block kb: rows 8 kb + lane / 8 (of K, or
  // of V^T), chunk lane % 8 fetching logical chunk (lane % 8) ^ ((r / 2) % 8).
  const int k_r0 = lane >> 3;
  auto koff = [&](int kb) -> uint32_t {
    const int r = kb * 8 + k_r0;
    return (uint32_t)r * D + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4);
  };
  auto voff = [&](int kb) -> uint32_t {
    const int r = kb * 8 + k_r0;
    return (uint32_t)r * (uint32_t)npad * 2u + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4);
  };
  uint8_t* const kbuf0 = smem;
  uint8_t* const vbuf0 = smem + 2 * KBYTES;
  auto kbuf = [&](int t) { return kbuf0 + (t & 1) * KBYTES; };
  auto vbuf = [&](int t) { return vbuf0 + (t & 1) * VBYTES; };
  // all eight waves: K block `wave`, V blocks 2 wave and 2 wave + 1 of tile j
  const uint32_t k_all = koff(wave), v_all0 = voff(2 * wave), v_all1 = voff(2 * wave + 1);
  auto dma_k_all = [&](int j, uint8_t* buf) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(buf + wave * 1024), 16, k_all + (uint32_t)(j * BC) * D,
                                             0, 0, 0);
  };
  auto dma_v_all = [&](int j, uint8_t* buf) {
    const uint32_t row_off = (uint32_t)(j * BC) * 2u;          // tile j: keys 64 j.. of every row
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(buf + 2 * wave * 1024), 16, v_all0 + row_off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(buf + (2 * wave + 1) * 1024), 16, v_all1 + row_off, 0, 0,
                                             0);
  };

  // K operand addresses: row 32 G + ln, logical chunk 2 st + lh, swizzle
  // (ln / 2) % 8.
  uint32_t k_off[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) k_off[st] = (uint32_t)ln * D + (uint32_t)((((2 * st + lh) ^ ((ln >> 1) & 7))) << 4);
  // V^T operands: P V step k (key block G = k / 2, half cc = k % 2) reads
  // row 32 p + ln, logical chunk 4 G + 2 lh + cc (the prepass's key order
  // puts there the 8 keys of this lane's P^T chunk), swizzle (ln / 2) % 8.
  uint32_t vaddr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    vaddr[k] = (uint32_t)ln * VROW + (uint32_t)(((4 * (k >> 1) + 2 * lh + (k & 1)) ^ ((ln >> 1) & 7)) << 4);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;
  i32x16 si[2];                                  // S^T of the current tile (biased int32)
  u32x4 pb[2][2];                                // P^T operand of the pending P V, 8 keys per chunk
  u32x4 va[2][4];                                // V operands of P V step k in va[k % 2]

  auto vread = [&](const uint8_t* vb, auto kk) {
    constexpr int k = decltype(kk)::value;
#pragma unroll
    for (int p = 0; p < 4; ++p) va[k % 2][p] = *reinterpret_cast<const u32x4*>(vb + p * 32 * VROW + vaddr[k]);
  };
  auto vread_first = [&](const uint8_t* vb) { vread(vb, std::integral_constant<int, 0>{}); };

  // ---- MFMA phase: O^T += V^T P^T for the previous tile (four steps of 16
  // keys, four MFMAs each), then S^T = K Q^T for this one; the K operands
  // are read two per P V step, the V operands one step ahead (the first
  // step's already in va[0] when PRE).
  auto mma_phase = [&](const uint8_t* kb, const uint8_t* vb, auto do_pv, auto do_qk, auto pre_tag) {
    constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
    constexpr bool PRE = decltype(pre_tag)::value;
    u32x4 ka[8];                                  // chunk c = 2 st + G
    auto kread = [&](int c) {
      ka[c] = *reinterpret_cast<const u32x4*>(kb + 32 * (c & 1) * D + k_off[c >> 1]);
    };
    if constexpr (PV) {
      if constexpr (!PRE) vread(vb, std::integral_constant<int, 0>{});
      static_for<4>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k + 1 < 4) vread(vb, std::integral_constant<int, k + 1>{});
        if constexpr (QK) {
          kread(2 * k);
          kread(2 * k + 1);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[p] = mfma_chunk<T>(va[k % 2][p], pb[k >> 1][k & 1], acc[p]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (QK) {
#pragma unroll
      for (int c = 0; c < 8; ++c) kread(c);
    }
    if constexpr (QK) {
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) si[G][i] = kAccBias;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int G = 0; G < 2; ++G)
          si[G] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, ka[2 * st + G]),
                                                        __builtin_bit_cast(i32x4, qreg[st]), si[G], 0, 0, 0);
    }
  };

  // ---- softmax phase for tile t: S -> 16-bit P^T (pb), m, l, rescale.  The
  // MASKED form is the ragged last tile (keys at or past n_eff drop out).
  float sk_next = skh[0];
  auto softmax_phase = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const float c = sq_w * sk_next * c_log2;      // one K scale block per tile
    sk_next = skh[min(t + 1, groups - 1)];        // the next tile's, a phase pair ahead
    float s[32];
    float mx;
    if constexpr (MASKED) {
      const int kv0 = t * BC;
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + 32 * G + 8 * (i >> 2) + 4 * lh + (i & 3);
          if constexpr (SQ)                       // table in log2 units; -inf past n_eff
            s[16 * G + i] = __builtin_fmaf(unbias(si[G][i]), c, mk[16 * G + i]);
          else if constexpr (kAdd)                // keys past N read -inf
            s[16 * G + i] = __builtin_fmaf(unbias(si[G][i]), c, mk[16 * G + i] * kLog2e);
          else
            s[16 * G + i] = key < n_eff ? unbias(si[G][i]) * c : -INFINITY;
        }
      mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 32; ++i) mx = fmaxf(mx, s[i]);
    } else {
      // the max of the exact integer-valued floats, scaled once (c >= 0);
      // four independent chains (a single wave issues this phase)
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[16 * G + i] = unbias(si[G][i]);
      float mq[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
      for (int i = 4; i < 32; ++i) mq[i & 3] = fmaxf(mq[i & 3], s[i]);
      mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])) * c;
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
    // P = exp2(s - m) <= 1, rounded to the 16-bit type for the P V operand;
    // the row sum of the unrounded P in four partial sums
    float ps[4] = {-0.f, -0.f, -0.f, -0.f};       // -0 + x == x: the first adds fold away
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = s[16 * G + 8 * cc + e];
          pv[e] = MASKED ? __builtin_amdgcn_exp2f(x - m_use) : __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m_use));
          ps[e & 3] += pv[e];
        }
        pb[G][cc] = pack_chunk<T>(pv);
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // the phase's results exist before its closing barrier
    asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(l_run), "v"(m_run));
  };

  if (nt > 0) {
    dma_k_all(0, kbuf0);                          // prologue: K(0) by all eight waves
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
    __syncthreads();
    // Tile DMA: group A loads K tiles (blocks 2 (w % 4), 2 (w % 4) + 1), group
    // B V tiles (blocks 4 (w % 4) .. + 3), from offsets computed once (tile j
    // adds j BC rows).
    const int w4 = wave & 3;
    uint32_t offs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) offs[i] = grp == 0 ? (i < 2 ? koff(2 * w4 + i) : 0u) : voff(4 * w4 + i);
    auto dma_k = [&](uint8_t* buf, int j) {
      const uint32_t row_off = (uint32_t)(j * BC) * D;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(buf + (2 * w4 + i) * 1024), 16, offs[i] + row_off, 0,
                                                 0, 0);
    };
    auto dma_v = [&](uint8_t* buf, int j) {
      const uint32_t row_off = (uint32_t)(j * BC) * 2u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(buf + (4 * w4 + i) * 1024), 16, offs[i] + row_off, 0,
                                                 0, 0);
    };
    pp_phase_loop(
        grp, nt,
        [&](int tk, int tv, auto pv, auto qk, auto pre) {
          if constexpr (kRowTerm && decltype(qk)::value) load_mask_tile<2>(mk, mrow, mstride, mvec, tk * BC, n_eff, lh);
          mma_phase(kbuf(tk), vbuf(tv), pv, qk, pre);
        },
        [&](int t) { softmax_phase(t, BoolTag<kRowTerm>{}); }, [&](int t) { dma_k(kbuf(t), t); },
        [&](int t) { dma_v(vbuf(t), t); }, [&](int t) { vread_first(vbuf(t)); });
  }
  // The ragged last tile, all eight waves in step, after every full tile
  // (both groups have passed barrier 2nt + 1, so every buffer is free).
  if (nt < ntiles) {
    dma_k_all(nt, kbuf0);
    dma_v_all(nt, vbuf0);
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
    __syncthreads();
    if constexpr (kRowTerm) load_mask_tile<2>(mk, mrow, mstride, mvec, nt * BC, n_eff, lh);
    mma_phase(kbuf0, vbuf0, BoolTag<false>{}, BoolTag<true>{}, BoolTag<false>{});
    softmax_phase(nt, BoolTag<true>{});
    mma_phase(kbuf0, vbuf0, BoolTag<true>{}, BoolTag<false>{}, BoolTag<false>{});
  }

  const float l_tot = wave_sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = O + ((size_t)bh * N + q_row) * D;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * p + 8 * g + 4 * lh;
        store4<T>(orow + d0, acc[p][4 * g] * inv, acc[p][4 * g + 1] * inv, acc[p][4 * g + 2] * inv,
                  acc[p][4 * g + 3] * inv);
      }
    if (LSE != nullptr && lh == 0)
      LSE[(size_t)bh * N + q_row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// The 16-bit-PV form: every mask, with or without Q smoothing.
template <typename T>
int launch_int8qk_pv16(const void* q, const void* k, const void* v, void* o, float* lse, int mask_kind, MaskArgs m,
                       int B, int H, int N, float scale, void* workspace, const Int8Layout& L, bool smooth,
                       hipStream_t st) {
  const Int8Ops op = int8_prepass<T, true>(q, k, v, B, H, N, scale, workspace, L, smooth, st);
  const int nqt = (N + 255) / 256;
  const T* vt = static_cast<const T*>(op.vt);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(B * H * nqt), dim3(512), 0, st, op.q8, op.k8, vt, op.sq, op.sk, op.comp, m,
                       static_cast<T*>(o), lse, H, N, L.npad, L.groups, nqt, scale * kLog2e);
  };
  if (smooth) {   // additive masks are refused with Q smoothing (host check)
    if (mask_kind == kMaskLen) go(fa_int8qk_pv16_pp_kernel<T, kMaskLen, true>);
    else go(fa_int8qk_pv16_pp_kernel<T, kMaskNone, true>);
  } else if (mask_kind == kMaskLen) {
    go(fa_int8qk_pv16_pp_kernel<T, kMaskLen, false>);
  } else if (mask_kind == kMaskAdd) {
    go(fa_int8qk_pv16_pp_kernel<T, kMaskAdd, false>);
  } else {
    go(fa_int8qk_pv16_pp_kernel<T, kMaskNone, false>);
  }
  return FA_OK;
}

}  // namespace fa
