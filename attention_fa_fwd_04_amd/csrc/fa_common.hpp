// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers over 16-byte operand chunks, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float    f32x2  __attribute__((ext_vector_type(2)));
typedef float    f32x4  __attribute__((ext_vector_type(4)));
typedef float    f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t  i32x4  __attribute__((ext_vector_type(4)));
typedef int32_t  i32x8  __attribute__((ext_vector_type(8)));
typedef int32_t  i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2  __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4  __attribute__((ext_vector_type(4)));
typedef __bf16   bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2  __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8  __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum MaskKind { kMaskNone = 0, kMaskAdd = 1, kMaskLen = 2 };

struct MaskArgs {
  const void* ptr;
  int64_t sb, sh, sq, sk;
};

// True when every query row of the mask is key-contiguous and 16-byte aligned
// (the same for all lanes: it depends on the kernel arguments only).
__device__ __forceinline__ bool mask_rows_vec4(const MaskArgs& m) {
  return m.sk == 1 && ((m.sb | m.sh | m.sq) & 3) == 0 && (reinterpret_cast<uintptr_t>(m.ptr) & 15) == 0;
}

// Additive-mask values (as stored) of one lane's keys of the key tile at kv0
// (SB blocks of 32 keys): index 16 G + i holds key kv0 + 32 G + 8 (i >> 2) +
// 4 lh + (i & 3), the order of the transposed score tile.  Keys at or past nk
// read -inf.  A whole tile of a vec4 mask row takes 4 SB 16-byte loads,
// anything else one load per key.  Issued a tile ahead of their use, the
// loads complete under the current tile's work.
template <int SB>
__device__ __forceinline__ void load_mask_tile(float (&dst)[16 * SB], const float* mrow, int64_t sk, bool vec4,
                                               int kv0, int nk, int lh) {
  if (vec4 && kv0 + 32 * SB <= nk) {
#pragma unroll
    for (int G = 0; G < SB; ++G)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(mrow + kv0 + 32 * G + 8 * g + 4 * lh);
        dst[16 * G + 4 * g] = x.x;
        dst[16 * G + 4 * g + 1] = x.y;
        dst[16 * G + 4 * g + 2] = x.z;
        dst[16 * G + 4 * g + 3] = x.w;
      }
  } else {
#pragma unroll
    for (int G = 0; G < SB; ++G)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + 32 * G + 8 * (i >> 2) + 4 * lh + (i & 3);
        dst[16 * G + i] = key < nk ? mrow[(int64_t)key * sk] : -INFINITY;
      }
  }
}

// Additive-mask values (as stored) of the 4 consecutive keys key0 .. key0 + 3
// of one query row; keys at or past nk read -inf.  VEC: the row is
// key-contiguous and 16-byte aligned and all four keys are below nk, so one
// 16-byte load does.
template <bool VEC>
__device__ __forceinline__ f32x4 mask_quad(const float* mrow, int64_t sk, int key0, int nk) {
  if constexpr (VEC) {
    return *reinterpret_cast<const f32x4*>(mrow + key0);
  } else {
    f32x4 r;
    r.x = key0 < nk ? mrow[(int64_t)key0 * sk] : -INFINITY;
    r.y = key0 + 1 < nk ? mrow[(int64_t)(key0 + 1) * sk] : -INFINITY;
    r.z = key0 + 2 < nk ? mrow[(int64_t)(key0 + 2) * sk] : -INFINITY;
    r.w = key0 + 3 < nk ? mrow[(int64_t)(key0 + 3) * sk] : -INFINITY;
    return r;
  }
}

// Element strides of a [B, H, N, D] tensor whose D elements are contiguous:
// element (b, h, n, d) is at base[b * sb + h * sh + n * sn + d].
struct RowLayout {
  int64_t sb, sh, sn;
};

template <typename T> struct Elt;
template <> struct Elt<float>    { static constexpr int kBytes = 4; };
template <> struct Elt<_Float16> { static constexpr int kBytes = 2; };
template <> struct Elt<__bf16>   { static constexpr int kBytes = 2; };

// 32x32 MFMA accumulate over one 16-byte operand chunk per lane.  For the
// 16-bit types that is one 32x32x16 instruction (8 elements per lane); for
// float it is four 32x32x2 instructions, element e of each lane's chunk
// feeding instruction e.  A and B always take the same element of the same
// lane half, so any consistent assignment of the contraction index to
// (lane half, element) gives the same sum.
template <typename T> __device__ __forceinline__ f32x16 mfma_chunk(u32x4 a, u32x4 b, f32x16 c);

template <> __device__ __forceinline__ f32x16 mfma_chunk<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_chunk<_Float16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_chunk<float>(u32x4 a, u32x4 b, f32x16 c) {
  // Bit-cast whole vectors, then index: a bit-cast of a single ext-vector
  // element is not reliably lowered to that element.
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  const f32x4 bf = __builtin_bit_cast(f32x4, b);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.x, bf.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.y, bf.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.z, bf.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.w, bf.w, c, 0, 0, 0);
  return c;
}

// Two floats -> two 16-bit values in one dword (round to nearest even).
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Four floats -> four OCP e4m3fn bytes in one dword, round to nearest even
// (the hardware conversion of the quantised kernels, for 448 P and for V;
// inputs stay within +-448 (1 + 2^-22) there).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  // the first conversion fills the low half and keeps the old high half,
  // which the second overwrites: any old value will do, and a's own bits
  // (dead after this) let the conversion write in place of a
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// 16 bytes of operand from 16/sizeof(T) consecutive floats.
template <typename T> __device__ __forceinline__ u32x4 pack_chunk(const float* p) {
  u32x4 r;
  r.x = pack2<T>(p[0], p[1]);
  r.y = pack2<T>(p[2], p[3]);
  r.z = pack2<T>(p[4], p[5]);
  r.w = pack2<T>(p[6], p[7]);
  return r;
}
template <> __device__ __forceinline__ u32x4 pack_chunk<float>(const float* p) {
  const f32x4 v = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(u32x4, v);
}

// Four consecutive outputs.
template <typename T> __device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  u32x2 r = {pack2<T>(a, b), pack2<T>(c, d)};
  *reinterpret_cast<u32x2*>(dst) = r;
}
template <> __device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  f32x4 r = {a, b, c, d};
  *reinterpret_cast<f32x4*>(dst) = r;
}

// Logical tile for a workgroup.  Consecutive workgroup ids are dealt round
// robin to the 8 XCDs; this remap hands each XCD one contiguous run of
// logical tiles, so the query tiles of a head (which re-read the same K/V)
// run on the same XCD and share its L2.  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, k = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// Buffer resource over [base, base + bytes): loads at offsets outside the
// range return zero instead of touching memory, so tails and masked rows
// need no branches.
// LDS destination pointer of the buffer-load-to-LDS builtin.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOobOffset = 0x80000000u;   // beyond any range this library builds

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Combine a value with the same lane of the other wave half (lane ^ 32).
__device__ __forceinline__ float wave_max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  return x + __shfl_xor(x, 32);
}
// The same max through v_permlane32_swap: swap(v, v) leaves {own, other
// half's} value in its two results on every lane (in either order), a VALU
// exchange with no trip through the LDS crossbar, and max is symmetric in
// the pair, so both halves get the same result.  Used where the exchange
// is on every tile's critical path (the quantised kernel's exact row max);
// the D = 128 16-bit kernels keep the crossbar form, which the register
// allocator handles better in their tile loops.
__device__ __forceinline__ float wave_max_halves_valu(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

}  // namespace fa
