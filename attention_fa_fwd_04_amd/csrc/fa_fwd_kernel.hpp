// Attention forward kernel for gfx950 (fp32 / fp16 / bf16).
//
// Method: handbook page "算子加速：注意力、编译与融合", section
// "注意力：从 O(N²) 显存到分块" (figure and blocked code): for each query tile,
// stream K/V tiles through on-chip memory, form the score tile, update the
// running row max m and denominator l, rescale the accumulator by
// exp(m_old - m_new) and add P V; only O (and the row log-sum-exp) is written.
//
// Work split.  A workgroup is 4 waves and owns 128 consecutive query rows of
// one (b, h) head; wave w owns rows 32w..32w+31.  Each wave computes the
// transposed score tile S^T = K Q^T with 32x32 MFMAs (keys on the M side,
// queries on the N side), so lane (n, h) = (lane % 32, lane / 32) holds query
// n and, per 32-key block, the 16 keys 8g + 4h + r (g, r in 0..3) in
// accumulator register 4g + r.  The softmax is then lane-local: a row max
// needs one exchange with the other lane half, the row sum is kept per lane
// half and added once at the end.
//
// The output is accumulated transposed too, O^T += V^T P^T, so the running
// rescale by alpha = exp2(m_old - m_new) touches only the lane's own query.
// The P^T operand is the lane's own scores (no data movement); the V^T
// operand needs, per lane, consecutive keys at a fixed channel, so the V tile
// is transposed on its way into LDS and its key order permuted within each
// 32-key block (key 8g + 4h + r stored at position 16h + 4g + r), which makes
// each lane's 16 keys contiguous and 16-byte readable.
//
// Memory path.  K rows go to LDS as-is (row stride odd in 16-byte units, which
// keeps the 16-lane phases of ds_read_b128 on distinct banks); V goes through
// registers, is transposed with byte permutes and written as V^T.  The next
// K/V tile is fetched into registers while the current one is consumed, and
// written to the other half of a double buffer afterwards: one barrier per
// tile.  Q stays in registers in MFMA operand layout for the whole loop.
//
// Exponentials are exp2 with scale*log2(e) folded into the FMA that subtracts
// the running max.  Key tails (N % 64) and key-length masks drop keys on the
// boundary tile only; tiles wholly past the key length are never visited.
#pragma once

#include "fa_common.hpp"

namespace fa {

template <typename T, int D, int BC, int MASK, int NW>
struct FwdCfg {
  static constexpr int E = Elt<T>::kBytes;
  static constexpr int EPC = 16 / E;              // elements per 16-byte chunk
  static constexpr int DCH = D * E / 16;          // chunks per row
  static constexpr int QKS = (DCH + 1) / 2;       // MFMA steps over D (2 chunks each)
  // K row stride in LDS, bytes.  A row of an odd number of chunks is stored
  // unpadded: the stride (odd in 16-byte units) keeps the 16-lane phases of
  // both the row-per-lane operand reads and the consecutive staging stores on
  // distinct banks.  The QK step that would read chunk DCH (past the row)
  // re-reads chunk DCH - 1 instead; its Q chunk is zero, so it adds nothing.
  // Even chunk counts keep a padded row (16 bytes past the last QK step).
  static constexpr bool KDENSE = (DCH & 1) != 0;
  static constexpr int KSTR = KDENSE ? 16 * DCH : 32 * QKS + 16;
  static constexpr int PVB = (D + 31) / 32;       // 32-channel blocks of O^T
  static constexpr int VSTR = BC * E + 16;        // V^T row stride in LDS, bytes
  static constexpr int KBYTES = BC * KSTR;
  static constexpr int VBYTES = 32 * PVB * VSTR;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int SB = BC / 32;              // 32-key blocks per tile
  static constexpr int NT = 64 * NW;              // threads per workgroup
  static constexpr int BR = 32 * NW;              // query rows per workgroup
  static constexpr int KITEMS = BC * DCH;
  static constexpr int KIT = (KITEMS + NT - 1) / NT;
  static constexpr int VITEMS = (BC / 4) * DCH;
  static constexpr int VIT = (VITEMS + NT - 1) / NT;
  static_assert(D * E % 16 == 0, "rows must be whole 16-byte chunks");
  static_assert(BC % 32 == 0, "key tile must be whole 32-key blocks");
  static_assert(2 * BUF <= 160 * 1024, "double buffer must fit in LDS");
};

template <bool B> struct BoolTag { static constexpr bool value = B; };

// ONE_TILE: every key fits in one tile (Nk <= BC, guaranteed by the caller):
// one LDS buffer and no prefetch, so more workgroups fit on a CU (batched
// short windows).
template <typename T, int D, int BC, int MASK, int NW, int MINB, bool ONE_TILE = false>
__global__ __launch_bounds__(64 * NW, MINB) void fa_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, MaskArgs mask,
    RowLayout lq, RowLayout lk, RowLayout lv, RowLayout lo,
    int H, int Nq, int Nk, int nqt, float c_log2) {
  using C = FwdCfg<T, D, BC, MASK, NW>;
  constexpr int NBUF = ONE_TILE ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int b = bh / H, h = bh - b * H;
  // Row pitches in bytes (D contiguous; validated to fit the 32-bit ranges).
  const uint32_t qs = (uint32_t)(lq.sn * C::E), ks = (uint32_t)(lk.sn * C::E), vs = (uint32_t)(lv.sn * C::E);

  int n_eff = Nk;
  if constexpr (MASK == kMaskLen) {
    const int L = reinterpret_cast<const int*>(mask.ptr)[b];
    n_eff = L < 0 ? 0 : (L > Nk ? Nk : L);
  }
  const int ntiles = (n_eff + BC - 1) / BC;
  // Rows at or past n_eff read as zero: K and V ranges end there.
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + b * lq.sb + h * lq.sh, (uint32_t)Nq * qs);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + b * lk.sb + h * lk.sh, (uint32_t)n_eff * ks);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + b * lv.sb + h * lv.sh, (uint32_t)n_eff * vs);

  const int q_row = qt * C::BR + wave * 32 + ln;
  const bool q_ok = q_row < Nq;

  // Q in B-operand layout: step s, lane half h holds chunk 2s + h of its row
  // (chunks past D, and rows past N, read as zero).
  u32x4 qreg[C::QKS];
#pragma unroll
  for (int s = 0; s < C::QKS; ++s) {
    const int ch = 2 * s + lh;
    qreg[s] = buf_load16(qr, ch < C::DCH ? (uint32_t)q_row * qs + ch * 16 : kOobOffset);
  }

  // Zero the padding the tile writes never touch: K chunks past D (QK steps
  // are 2 chunks wide) and V^T rows past D (PV blocks are 32 channels).
  if constexpr (!C::KDENSE && 2 * C::QKS > C::DCH) {
    for (int r = tid; r < NBUF * BC; r += C::NT) {
      uint8_t* p = smem + (r / BC) * C::BUF + (r % BC) * C::KSTR + C::DCH * 16;
      for (int c = 0; c < (2 * C::QKS - C::DCH) * 16; c += 16)
        *reinterpret_cast<u32x4*>(p + c) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (32 * C::PVB > D) {
    constexpr int rows = 32 * C::PVB - D;
    constexpr int chunks = BC * C::E / 16;
    for (int it = tid; it < NBUF * rows * chunks; it += C::NT) {
      const int buf = it / (rows * chunks), rem = it % (rows * chunks);
      uint8_t* p = smem + buf * C::BUF + C::KBYTES + (D + rem / chunks) * C::VSTR + (rem % chunks) * 16;
      *reinterpret_cast<u32x4*>(p) = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- tile staging (global -> registers -> LDS) ----
  u32x4 kst[C::KIT];
  u32x4 vst[C::VIT][4];

  // Loads past the last tile read zeros (outside the buffer range), so the
  // prefetch needs no guard.
  auto load_tile = [&](int j) {
    const uint32_t row0 = (uint32_t)(j * BC);
#pragma unroll
    for (int i = 0; i < C::KIT; ++i) {
      const int it = tid + i * C::NT;
      const uint32_t row = row0 + it / C::DCH, c = it % C::DCH;
      kst[i] = buf_load16(kr, (C::KITEMS % C::NT == 0 || it < C::KITEMS) ? row * ks + c * 16 : kOobOffset);
    }
#pragma unroll
    for (int i = 0; i < C::VIT; ++i) {
      const int it = tid + i * C::NT;
      const int kg = it % (BC / 4), dc = it / (BC / 4);
      const bool ok = C::VITEMS % C::NT == 0 || it < C::VITEMS;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vst[i][r] = buf_load16(vr, ok ? (row0 + 4 * kg + r) * vs + dc * 16 : kOobOffset);
    }
  };

  auto store_tile = [&](int buf) {
    uint8_t* kb = smem + buf * C::BUF;
    uint8_t* vb = kb + C::KBYTES;
#pragma unroll
    for (int i = 0; i < C::KIT; ++i) {
      const int it = tid + i * C::NT;
      if (C::KITEMS % C::NT == 0 || it < C::KITEMS) {
        const int row = it / C::DCH, c = it - row * C::DCH;
        *reinterpret_cast<u32x4*>(kb + row * C::KSTR + c * 16) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::VIT; ++i) {
      const int it = tid + i * C::NT;
      if (!(C::VITEMS % C::NT == 0 || it < C::VITEMS)) continue;
      const int kg = it % (BC / 4), dc = it / (BC / 4);
      const int key = 4 * kg;                       // first of 4 consecutive keys
      const int kk = key & 31;
      const int pos = (key & ~31) + 16 * ((kk >> 2) & 1) + 4 * (kk >> 3);
      uint8_t* base = vb + pos * C::E;
      if constexpr (C::E == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w = {vst[i][0][e], vst[i][1][e], vst[i][2][e], vst[i][3][e]};
          *reinterpret_cast<u32x4*>(base + (dc * 4 + e) * C::VSTR) = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x2 w;
          w.x = __builtin_amdgcn_perm(vst[i][1][e >> 1], vst[i][0][e >> 1], sel);
          w.y = __builtin_amdgcn_perm(vst[i][3][e >> 1], vst[i][2][e >> 1], sel);
          *reinterpret_cast<u32x2*>(base + (dc * 8 + e) * C::VSTR) = w;
        }
      }
    }
  };

  // Running state.  m_run is the reference the exponentials are taken
  // against (log2 units); it is raised only when some row's max exceeds it
  // by more than kLazy, so P <= 2^kLazy and the accumulator is rescaled
  // rarely.  Normalising by l at the end makes the result independent of
  // the reference.
  constexpr float kLazy = 8.f;
  float m_run = -INFINITY;
  float l_run = 0.f;         // this lane half's share of the denominator
  f32x16 acc[C::PVB];
#pragma unroll
  for (int p = 0; p < C::PVB; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;

  // Additive masks are scaled to log2 units before the max; otherwise the
  // scale is folded into the exp2 argument.
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

  // One K/V tile: scores, online softmax, P V.  MASKED adds the additive
  // mask or drops keys at or past n_eff; it is only needed on the last tile
  // unless the mask is additive.
  auto step = [&](int j, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = ONE_TILE ? 0 : (j & 1);
    if constexpr (!ONE_TILE) load_tile(j + 1);
    const uint8_t* kb = smem + buf * C::BUF;
    const uint8_t* vb = kb + C::KBYTES;
    const int kv0 = j * BC;

    // S^T = K Q^T.  The K operand chunks of 32-key block G + 1 are read while
    // block G's MFMAs run; the scheduling barriers keep the compiler from
    // sinking those reads back next to their MFMAs, so LDS latency overlaps
    // the matrix work.
    f32x16 s[C::SB];
    u32x4 ka[C::QKS];
    auto kch = [&](int st) { return C::KDENSE ? min(2 * st + lh, C::DCH - 1) : 2 * st + lh; };
#pragma unroll
    for (int st = 0; st < C::QKS; ++st)
      ka[st] = *reinterpret_cast<const u32x4*>(kb + ln * C::KSTR + kch(st) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int G = 0; G < C::SB; ++G) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[G][i] = 0.f;
#pragma unroll
      for (int st = 0; st < C::QKS; ++st) {
        const u32x4 a = ka[st];
        if (G + 1 < C::SB)
          ka[st] = *reinterpret_cast<const u32x4*>(kb + (32 * (G + 1) + ln) * C::KSTR + kch(st) * 16);
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

    // P = exp2(S*c - m), row sum
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

    // O^T += V^T P^T
#pragma unroll
    for (int G = 0; G < C::SB; ++G) {
#pragma unroll
      for (int cc = 0; cc < 16 / C::EPC; ++cc) {
        float pv[C::EPC];
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) pv[e] = s[G][cc * C::EPC + e];
        const u32x4 bop = pack_chunk<T>(pv);
#pragma unroll
        for (int p = 0; p < C::PVB; ++p) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(
              vb + (32 * p + ln) * C::VSTR + (32 * G + 16 * lh + cc * C::EPC) * C::E);
          acc[p] = mfma_chunk<T>(a, bop, acc[p]);
        }
      }
    }

    if constexpr (!ONE_TILE) {
      store_tile(buf ^ 1);
      __syncthreads();
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  if constexpr (kPre) {
    for (int j = 0; j < ntiles; ++j) step(j, BoolTag<true>{});
  } else {
    const int nfull = n_eff / BC;
    for (int j = 0; j < nfull; ++j) step(j, BoolTag<false>{});
    if (nfull < ntiles) step(nfull, BoolTag<true>{});
  }

  // ---- epilogue: O = acc / l, lse = ln 2 * (m + log2 l) ----
  const float l_tot = wave_sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    T* orow = O + b * lo.sb + h * lo.sh + (int64_t)q_row * lo.sn;
#pragma unroll
    for (int p = 0; p < C::PVB; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * p + 8 * g + 4 * lh;
        if (d0 < D)
          store4<T>(orow + d0, acc[p][4 * g] * inv, acc[p][4 * g + 1] * inv,
                    acc[p][4 * g + 2] * inv, acc[p][4 * g + 3] * inv);
      }
    if (LSE != nullptr && lh == 0)
      LSE[(size_t)bh * Nq + q_row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace fa
