// INT8-QK / FP8-PV attention variant: workspace layout and launcher.
#pragma once

#include "fa_common.hpp"
#include "fa.h"

namespace fa {

constexpr int kInt8Bc = 64;        // keys per tile of the online softmax
constexpr int kQBlock = 64;        // tokens per INT8 scale block
constexpr int kStatRows = 512;     // tokens per partial-statistics workgroup
constexpr int kMaxSplits = 256;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets of the workspace regions (each 256-byte aligned).
struct Int8Layout {
  int npad;          // N rounded up to kQBlock
  int groups;        // npad / kQBlock
  int splits;        // token splits of the K-mean / V-absmax reduction
  size_t q8, k8, v8t, sq, sk, sv, kpart, vpart, kmean;
  size_t total;
};

inline Int8Layout int8qk_workspace_layout(int B, int H, int N, int D) {
  Int8Layout L{};
  const size_t bh = (size_t)B * H;
  L.npad = (N + kQBlock - 1) / kQBlock * kQBlock;
  L.groups = L.npad / kQBlock;
  L.splits = (N + kStatRows - 1) / kStatRows;
  if (L.splits > kMaxSplits) L.splits = kMaxSplits;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  L.q8 = take(bh * L.npad * D);                 // int8 [BH, npad, D]
  L.k8 = take(bh * L.npad * D);                 // int8 [BH, npad, D]
  L.v8t = take(bh * (size_t)D * L.npad);        // e4m3 [BH, D, npad], keys permuted per 64
  L.sq = take(bh * L.groups * 4);               // f32 [BH, groups]
  L.sk = take(bh * L.groups * 4);
  L.sv = take(bh * (size_t)D * 4);              // f32 [BH, D]
  L.kpart = take(bh * (size_t)L.splits * D * 4);  // f32 [BH, splits, D] partial sums of K
  L.vpart = take(bh * (size_t)L.splits * D * 4);  // f32 [BH, splits, D] partial max |V|
  L.kmean = take(bh * (size_t)D * 4);           // f32 [BH, D]
  L.total = off;
  return L;
}

template <typename T>
int launch_int8qk(const void*, const void*, const void*, void*, float*, const int*,
                  int, int, int, float, void*, const Int8Layout&, hipStream_t) {
  return FA_ERR_UNSUPPORTED;
}

}  // namespace fa
