// C ABI of libfa.so: host-side validation, kernel selection and launch.
// Declarations and conventions: include/fa.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fa.h"
#include "fa_fwd_kernel.hpp"
#include "fa_fwd_dma.hpp"
#include "fa_fwd_pp.hpp"
#include "fa_int8qk.hpp"
#include "fa_int8qk_pv16_pp.hpp"
#include "fa_merge.hpp"
#include "fa_probe.hpp"

// Tile configuration of fa_fwd_kernel (fp32, and 16-bit D = 32 / 40; 16-bit
// D = 128 runs fa_fwd_pp_kernel or fa_fwd_dma_kernel): D = 128 (fp32) runs
// 8-wave workgroups (256 query rows), the small head dims 4-wave workgroups
// (128 rows) over 64-key tiles; fp32 uses 32-key tiles.  Every configuration
// keeps two waves per SIMD.
template <typename T, int D, int MASK> struct TileCfg {
  static constexpr int NW = (D >= 128) ? 8 : 4;
  static constexpr int BC = (sizeof(T) == 4) ? 32 : ((MASK == fa::kMaskAdd || D < 128) ? 64 : 128);
  static constexpr int MINB = 8 / NW;
};

namespace {

thread_local char g_hip_err[256] = "";

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("FA_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

const char* dtype_name(int dt) {
  switch (dt) {
    case FA_F32: return "f32";
    case FA_F16: return "f16";
    case FA_BF16: return "bf16";
    default: return "?";
  }
}

int record_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    std::snprintf(g_hip_err, sizeof(g_hip_err), "%s: %s", what, hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Arguments common to both entry points.
int check_common(const void* q, const void* k, const void* v, void* o, const float* lse,
                 const fa_mask_t* mask, int B, int H, int N, int D, float scale) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return FA_ERR_SHAPE;
  const int64_t nqt = (N + 127) / 128;
  if ((int64_t)B * H * nqt > INT32_MAX) return FA_ERR_SHAPE;
  if ((int64_t)B * H * (int64_t)N > (int64_t)1 << 40) return FA_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;
  if (mask) {
    if (mask->kind != FA_MASK_NONE && mask->kind != FA_MASK_ADDITIVE && mask->kind != FA_MASK_KEYLEN)
      return FA_ERR_ARG;
    if (mask->kind != FA_MASK_NONE) {
      if (!mask->ptr) return FA_ERR_NULL;
      if (!aligned(mask->ptr, 4)) return FA_ERR_ALIGN;
    }
    if (mask->kind == FA_MASK_ADDITIVE &&
        (mask->stride_b < 0 || mask->stride_h < 0 || mask->stride_q < 0 || mask->stride_k < 0))
      return FA_ERR_ARG;
  }
  return FA_OK;
}

// Row layouts of q, k, v, o in that order.
struct Layouts {
  fa::RowLayout q, k, v, o;
};

// Short query sequences (16-bit, Nq <= 384: batched window attention, whose
// windows of 8x8 latents are 64 tokens, case-study page, section 3.2): one,
// two or four waves per workgroup (32, 64 or 128 query rows) so no wave idles
// on rows past Nq; several workgroups share a CU.  For D = 128 the four-wave
// form beats the 256-row phase-alternating kernel up to 384 query rows
// (measured; from 512 the latter is faster).
template <typename T, int D, int MASK, int NW, int BC, bool ONE_TILE>
int launch_short_cfg(const void* q, const void* k, const void* v, void* o, float* lse, fa::MaskArgs m,
                     const Layouts& L, int B, int H, int Nq, int Nk, float scale, hipStream_t st) {
  using C = fa::FwdCfg<T, D, BC, MASK, NW>;
  const int nqt = (Nq + C::BR - 1) / C::BR;
  const int64_t grid = (int64_t)B * H * nqt;
  if (grid > INT32_MAX) return FA_ERR_SHAPE;
  if (log_enabled())
    std::fprintf(stderr, "[fa] fa_fwd(short) D=%d mask=%d B=%d H=%d Nq=%d Nk=%d grid=%lld block=%d BR=%d BC=%d lds=%d\n",
                 D, MASK, B, H, Nq, Nk, (long long)grid, C::NT, C::BR, BC, (ONE_TILE ? 1 : 2) * C::BUF);
  hipLaunchKernelGGL((fa::fa_fwd_kernel<T, D, BC, MASK, NW, 2, ONE_TILE>), dim3((unsigned)grid), dim3(C::NT), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<T*>(o), lse, m, L.q, L.k, L.v, L.o, H, Nq, Nk, nqt, scale * fa::kLog2e);
  return record_launch("fa_fwd_kernel(short)");
}

template <typename T, int D, int MASK, int NW>
int launch_short(const void* q, const void* k, const void* v, void* o, float* lse, fa::MaskArgs m,
                 const Layouts& L, int B, int H, int Nq, int Nk, float scale, hipStream_t st) {
  // D < 128 with all keys in one 64-key tile (windows): one LDS buffer and
  // no prefetch registers, so more workgroups fit on a CU (576x8 windows of
  // 64, D = 40: 25.0 -> 18.9 us; for D = 128 it measured slower).  Otherwise
  // double-buffered tiles, of 32 keys for D = 128 (whose staging registers
  // would leave one wave per SIMD with 64).
  if constexpr (D < 128)
    if (Nk <= 64) return launch_short_cfg<T, D, MASK, NW, 64, true>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
  return launch_short_cfg<T, D, MASK, NW, (D >= 128 ? 32 : 64), false>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
}
constexpr int kShortRows = 384;

template <typename T, int D, int MASK>
int launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, fa::MaskArgs m,
               const Layouts& L, int B, int H, int Nq, int Nk, float scale, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // (D = 128 keeps two waves: one wave of it would hold a SIMD alone)
    if constexpr (D < 128)
      if (Nq <= 32) return launch_short<T, D, MASK, 1>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    if (Nq <= 64) return launch_short<T, D, MASK, 2>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    if (Nq <= kShortRows) return launch_short<T, D, MASK, 4>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
  }
  if constexpr (D == 128 && sizeof(T) == 2 && MASK != fa::kMaskAdd) {
    // 16-bit, D = 128, no score mask: the two wave groups of each SIMD
    // alternate between the MFMA and softmax phases, 8 waves x 64-key tiles
    using C = fa::DmaCfg<T, 64, 8>;
    const int nqt = (Nq + C::BR - 1) / C::BR;
    const int grid = B * H * nqt;
    if (log_enabled())
      std::fprintf(stderr, "[fa] fa_fwd(pp) D=%d mask=%d B=%d H=%d Nq=%d Nk=%d grid=%d block=%d BR=%d BC=64 lds=%d\n",
                   D, MASK, B, H, Nq, Nk, grid, C::NT, C::BR, 4 * C::TILE);
    hipLaunchKernelGGL((fa::fa_fwd_pp_kernel<T, 64, MASK, false>), dim3(grid), dim3(C::NT), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<T*>(o), lse, m, L.q, L.k, L.v, L.o, H, Nq, Nk, nqt, scale * fa::kLog2e,
                       fa::SplitArgs{nullptr, nullptr, 0, 0});
    return record_launch("fa_fwd_pp_kernel");
  } else if constexpr (D == 128 && sizeof(T) == 2) {
    // 16-bit, D = 128 with an additive mask: K/V staged by LDS DMA, 8 waves
    // in step over 64-key tiles (the mask values of a tile are read next to
    // their use; wider tiles exceed the register budget)
    constexpr int NW = 8, BC = 64, MINB = 1;
    using C = fa::DmaCfg<T, BC, NW>;
    const int nqt = (Nq + C::BR - 1) / C::BR;
    const int grid = B * H * nqt;
    if (log_enabled())
      std::fprintf(stderr, "[fa] fa_fwd(dma) D=%d mask=%d B=%d H=%d Nq=%d Nk=%d grid=%d block=%d BR=%d BC=%d lds=%d\n",
                   D, MASK, B, H, Nq, Nk, grid, C::NT, C::BR, BC, 4 * C::TILE);
    hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<T, BC, MASK, NW, MINB>), dim3(grid), dim3(C::NT), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<T*>(o), lse, m, L.q, L.k, L.v, L.o, H, Nq, Nk, nqt, scale * fa::kLog2e);
    return record_launch("fa_fwd_dma_kernel");
  } else {
    using TC = TileCfg<T, D, MASK>;
    using C = fa::FwdCfg<T, D, TC::BC, MASK, TC::NW>;
    const int nqt = (Nq + C::BR - 1) / C::BR;
    const int grid = B * H * nqt;
    if (log_enabled())
      std::fprintf(stderr, "[fa] fa_fwd dtype=%s D=%d mask=%d B=%d H=%d Nq=%d Nk=%d grid=%d block=%d BR=%d BC=%d lds=%d\n",
                   sizeof(T) == 4 ? "f32" : "f16/bf16", D, MASK, B, H, Nq, Nk, grid, C::NT, C::BR, TC::BC, 2 * C::BUF);
    hipLaunchKernelGGL((fa::fa_fwd_kernel<T, D, TC::BC, MASK, TC::NW, TC::MINB>), dim3(grid), dim3(C::NT), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<T*>(o), lse, m, L.q, L.k, L.v, L.o, H, Nq, Nk, nqt, scale * fa::kLog2e);
    return record_launch("fa_fwd_kernel");
  }
}

template <typename T, int D>
int dispatch_mask(int kind, const void* q, const void* k, const void* v, void* o, float* lse,
                  fa::MaskArgs m, const Layouts& L, int B, int H, int Nq, int Nk, float scale, hipStream_t st) {
  switch (kind) {
    case FA_MASK_NONE: return launch_fwd<T, D, fa::kMaskNone>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case FA_MASK_ADDITIVE: return launch_fwd<T, D, fa::kMaskAdd>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case FA_MASK_KEYLEN: return launch_fwd<T, D, fa::kMaskLen>(q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    default: return FA_ERR_ARG;
  }
}

template <typename T>
int dispatch_d(int D, int kind, const void* q, const void* k, const void* v, void* o, float* lse,
               fa::MaskArgs m, const Layouts& L, int B, int H, int Nq, int Nk, float scale, hipStream_t st) {
  switch (D) {
    case 32: return dispatch_mask<T, 32>(kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case 40: return dispatch_mask<T, 40>(kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case 128: return dispatch_mask<T, 128>(kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    default: return FA_ERR_UNSUPPORTED;
  }
}

}  // namespace

namespace {
Layouts contiguous_layouts(int H, int Nq, int Nk, int D) {
  const fa::RowLayout lq{(int64_t)H * Nq * D, (int64_t)Nq * D, D};
  const fa::RowLayout lk{(int64_t)H * Nk * D, (int64_t)Nk * D, D};
  return Layouts{lq, lk, lk, lq};
}

// Kernels form 32-bit byte offsets for rows up to one tile (or one query
// block) past the last: with this margin those offsets never wrap, so they
// fall outside the buffer range and read as zero.
constexpr int64_t kRowMargin = 256;

// A strided view: non-negative strides, 16-byte aligned rows and (b, h)
// bases, and every row offset within the 32-bit range of a buffer resource.
int check_layout(const fa_stride_t* s, int rows, int D, size_t elt, bool output) {
  if (!s) return FA_ERR_NULL;
  if (s->stride_b < 0 || s->stride_h < 0 || s->stride_n <= 0) return FA_ERR_ARG;
  if (output && s->stride_n < D) return FA_ERR_ARG;
  if ((s->stride_b * (int64_t)elt) % 16 || (s->stride_h * (int64_t)elt) % 16 ||
      (s->stride_n * (int64_t)elt) % 16)
    return FA_ERR_ALIGN;
  if ((int64_t)(rows + kRowMargin) * s->stride_n * (int64_t)elt > (int64_t)UINT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse,
               const fa_mask_t* mask, int B, int H, int Nq, int Nk, int D, float scale,
               fa_dtype_t dtype, const Layouts& L, void* hip_stream) {
  int rc = check_common(q, k, v, o, lse, mask, B, H, Nq, D, scale);
  if (rc != FA_OK) return rc;
  if (Nk <= 0 || (int64_t)B * H * (int64_t)Nk > (int64_t)1 << 40) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (D != 32 && D != 40 && D != 128) return FA_ERR_UNSUPPORTED;
  const int kind = mask ? mask->kind : FA_MASK_NONE;
  fa::MaskArgs m{nullptr, 0, 0, 0, 0};
  if (kind != FA_MASK_NONE) m = fa::MaskArgs{mask->ptr, mask->stride_b, mask->stride_h, mask->stride_q, mask->stride_k};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  switch (dtype) {
    case FA_F32: return dispatch_d<float>(D, kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case FA_F16: return dispatch_d<_Float16>(D, kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    case FA_BF16: return dispatch_d<__bf16>(D, kind, q, k, v, o, lse, m, L, B, H, Nq, Nk, scale, st);
    default: return FA_ERR_UNSUPPORTED;
  }
}

size_t dtype_bytes(int dt) { return dt == FA_F32 ? 4 : 2; }

int contiguous_range_ok(int Nq, int Nk, int D, int dt) {
  const int64_t e = (int64_t)dtype_bytes(dt);
  return (int64_t)(Nq + kRowMargin) * D * e <= (int64_t)UINT32_MAX &&
         (int64_t)(Nk + kRowMargin) * D * e <= (int64_t)UINT32_MAX;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The even key-tile split of fa_fwd_pp_kernel (16-bit, D = 128, no mask,
// N a multiple of the 64-key tile): one workgroup per CU, used when whole
// query blocks would fill the last round of workgroups to less than 90 % and
// every workgroup still covers at least one block's worth of tiles (so a
// block is split at most once).
struct SplitPlan {
  int grid = 0;           // 0: the plain launch
  int nqt = 0, tiles = 0;
  int64_t units = 0;
  size_t bytes = 0;       // workspace
};
constexpr int kSplitBR = 256, kSplitBC = 64;

SplitPlan split_plan(int B, int H, int N, int D, int dtype, int mask_kind) {
  SplitPlan p;
  if ((dtype != FA_F16 && dtype != FA_BF16) || D != 128 || mask_kind != FA_MASK_NONE) return p;
  if (B <= 0 || H <= 0 || N <= 0 || N % kSplitBC != 0) return p;
  if (N <= kShortRows) return p;               // short sequences: the one/two/four-wave workgroups
  const int G = cu_count();
  if (G <= 0) return p;
  const int nqt = (N + kSplitBR - 1) / kSplitBR;
  const int64_t jobs = (int64_t)B * H * nqt;
  if (jobs < G) return p;
  const int64_t rounds = (jobs + G - 1) / G;
  if (jobs * 10 >= rounds * G * 9) return p;   // the last round is >= 90 % full
  p.grid = G;
  p.nqt = nqt;
  p.tiles = (N + kSplitBC - 1) / kSplitBC;
  p.units = jobs * p.tiles;
  // segments per workgroup: whole blocks of its range plus two split parts
  if ((p.units + G - 1) / G / p.tiles + 3 > fa::kMaxSegments) return SplitPlan{};
  const size_t cnt_bytes = ((size_t)(G + 1) * sizeof(unsigned) + 255) / 256 * 256;
  p.bytes = cnt_bytes + (size_t)(G + 1) * 2 * fa::kPartFloats * sizeof(float);
  return p;
}

template <typename T>
int launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                 float scale, const SplitPlan& p, void* workspace, hipStream_t st) {
  using C = fa::DmaCfg<T, kSplitBC, 8>;
  static_assert(C::BR == kSplitBR, "query block of the split launch");
  const Layouts L = contiguous_layouts(H, N, N, 128);
  const size_t cnt_bytes = ((size_t)(p.grid + 1) * sizeof(unsigned) + 255) / 256 * 256;
  fa::SplitArgs sk{static_cast<unsigned*>(workspace),
                   reinterpret_cast<float*>(static_cast<char*>(workspace) + cnt_bytes), p.units, p.tiles};
  if (log_enabled())
    std::fprintf(stderr, "[fa] fa_fwd_ws(pp, split) B=%d H=%d N=%d blocks=%lld tiles=%d grid=%d ws=%zu\n",
                 B, H, N, (long long)B * H * p.nqt, p.tiles, p.grid, p.bytes);
  const fa::MaskArgs m{nullptr, 0, 0, 0, 0};
  hipLaunchKernelGGL((fa::fa_fwd_pp_kernel<T, kSplitBC, fa::kMaskNone, true>), dim3(p.grid), dim3(C::NT), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<T*>(o), lse, m, L.q, L.k, L.v, L.o, H, N, N, p.nqt, scale * fa::kLog2e, sk);
  return record_launch("fa_fwd_pp_kernel(split)");
}
}  // namespace

// ---------------------------------------------------------------- static scratch
//
// fa_fwd_ws_static runs fa_fwd_ws's split launch on a library-owned scratch
// buffer instead of a caller workspace, for callers that cannot allocate
// device memory.  The split workspace depends only on the number of
// workgroups (one per CU), so one array sized for kStaticMaxGrid CUs serves
// every shape.  Each GPU the library runs on holds its own copy of the array
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device.
namespace {
constexpr int kStaticMaxGrid = 256;                                    // MI355X compute units
constexpr size_t kStaticCntBytes = ((size_t)(kStaticMaxGrid + 1) * sizeof(unsigned) + 255) / 256 * 256;
constexpr size_t kStaticScratchBytes =
    kStaticCntBytes + (size_t)(kStaticMaxGrid + 1) * 2 * fa::kPartFloats * sizeof(float);   // 69,477,632
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
__global__ __launch_bounds__(256) void fa_clear_u32_kernel(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct StaticScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
StaticScratchSlot g_static_scratch[kMaxDevices];

// Device address of the current device's scratch array.  The first call on a
// device looks the address up and queues a clear of the arrival counters on
// `st` (a fill kernel: the split protocol leaves them at zero after every
// completed call, so once per device is enough).
int static_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    std::snprintf(g_hip_err, sizeof(g_hip_err), "fa_fwd_ws_static: no usable current device (%d)", dev);
    return FA_ERR_HIP;
  }
  StaticScratchSlot& slot = g_static_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
      const int n = (int)(kStaticCntBytes / sizeof(unsigned));
      hipLaunchKernelGGL(fa_clear_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, static_cast<unsigned*>(p), n);
      e = hipGetLastError();
    }
    slot.err = e;
    slot.ptr = e == hipSuccess ? p : nullptr;
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr) {
    std::snprintf(g_hip_err, sizeof(g_hip_err), "fa_fwd_ws_static: scratch set-up on device %d: %s", dev,
                  hipGetErrorString(slot.err));
    return FA_ERR_HIP;
  }
  *out = slot.ptr;
  return FA_OK;
}
}  // namespace

extern "C" {

FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           const fa_mask_t* mask, int B, int H, int N, int D, float scale,
           fa_dtype_t dtype, void* hip_stream) {
  return fa_fwd_cross(q, k, v, o, lse, mask, B, H, N, N, D, scale, dtype, hip_stream);
}

FA_API int fa_fwd_cross(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_mask_t* mask, int B, int H, int Nq, int Nk, int D, float scale,
                        fa_dtype_t dtype, void* hip_stream) {
  if (Nq > 0 && Nk > 0 && D > 0 && !contiguous_range_ok(Nq, Nk, D, dtype)) return FA_ERR_SHAPE;
  return fwd_common(q, k, v, o, lse, mask, B, H, Nq, Nk, D, scale, dtype,
                    contiguous_layouts(H, Nq, Nk, D), hip_stream);
}

FA_API int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                          const fa_mask_t* mask, int B, int H, int Nq, int Nk, int D,
                          const fa_stride_t* q_strides, const fa_stride_t* k_strides,
                          const fa_stride_t* v_strides, const fa_stride_t* o_strides,
                          float scale, fa_dtype_t dtype, void* hip_stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || D <= 0) return FA_ERR_SHAPE;
  const size_t e = dtype_bytes(dtype);
  int rc;
  if ((rc = check_layout(q_strides, Nq, D, e, false)) != FA_OK) return rc;
  if ((rc = check_layout(k_strides, Nk, D, e, false)) != FA_OK) return rc;
  if ((rc = check_layout(v_strides, Nk, D, e, false)) != FA_OK) return rc;
  if ((rc = check_layout(o_strides, Nq, D, e, true)) != FA_OK) return rc;
  auto rl = [](const fa_stride_t* s) { return fa::RowLayout{s->stride_b, s->stride_h, s->stride_n}; };
  const Layouts L{rl(q_strides), rl(k_strides), rl(v_strides), rl(o_strides)};
  return fwd_common(q, k, v, o, lse, mask, B, H, Nq, Nk, D, scale, dtype, L, hip_stream);
}

FA_API size_t fa_fwd_workspace_bytes(int B, int H, int N, int D, fa_dtype_t dtype) {
  return split_plan(B, H, N, D, dtype, FA_MASK_NONE).bytes;
}

FA_API int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                     const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                     fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const int kind = mask ? mask->kind : FA_MASK_NONE;
  const SplitPlan p = split_plan(B, H, N, D, dtype, kind);
  if (p.grid == 0)
    return fa_fwd(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream);
  int rc = check_common(q, k, v, o, lse, mask, B, H, N, D, scale);
  if (rc != FA_OK) return rc;
  if (!contiguous_range_ok(N, N, D, dtype)) return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.bytes) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (dtype == FA_BF16) return launch_split<__bf16>(q, k, v, o, lse, B, H, N, scale, p, workspace, st);
  return launch_split<_Float16>(q, k, v, o, lse, B, H, N, scale, p, workspace, st);
}

FA_API int fa_fwd_ws_static(const void* q, const void* k, const void* v, void* o, float* lse,
                            const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                            fa_dtype_t dtype, void* hip_stream) {
  const int kind = mask ? mask->kind : FA_MASK_NONE;
  const SplitPlan p = split_plan(B, H, N, D, dtype, kind);
  if (p.grid == 0)
    return fa_fwd(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream);
  int rc = check_common(q, k, v, o, lse, mask, B, H, N, D, scale);
  if (rc != FA_OK) return rc;
  if (!contiguous_range_ok(N, N, D, dtype)) return FA_ERR_SHAPE;
  if (p.bytes > kStaticScratchBytes) {
    std::snprintf(g_hip_err, sizeof(g_hip_err),
                  "fa_fwd_ws_static: the split needs %zu bytes (%d CUs), the static scratch holds %zu (%d CUs)",
                  p.bytes, p.grid, kStaticScratchBytes, kStaticMaxGrid);
    return FA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  void* ws = nullptr;
  if ((rc = static_scratch(st, &ws)) != FA_OK) return rc;
  if (dtype == FA_BF16) return launch_split<__bf16>(q, k, v, o, lse, B, H, N, scale, p, ws, st);
  return launch_split<_Float16>(q, k, v, o, lse, B, H, N, scale, p, ws, st);
}

FA_API size_t fa_fwd_int8qk_workspace_bytes(int B, int H, int N, int D) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return 0;
  return fa::int8qk_workspace_layout(B, H, N, D).total;
}

FA_API size_t fa_fwd_int8qk_pv16_workspace_bytes(int B, int H, int N, int D) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return 0;
  return fa::int8qk_workspace_layout(B, H, N, D, true).total;
}

FA_API size_t fa_fwd_int8qk_smooth_workspace_bytes(int B, int H, int N, int D, int pv16) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || (pv16 != 0 && pv16 != 1)) return 0;
  return fa::int8qk_workspace_layout(B, H, N, D, pv16 != 0, true).total;
}

}  // extern "C"

namespace {
int int8qk_common(bool pv16, bool smooth, const void* q, const void* k, const void* v, void* o, float* lse,
                  const fa_mask_t* mask, int B, int H, int N, int D, float scale, fa_dtype_t dtype,
                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  const char* name = smooth ? "fa_fwd_int8qk_smooth" : pv16 ? "fa_fwd_int8qk_pv16" : "fa_fwd_int8qk";
  int rc = check_common(q, k, v, o, lse, mask, B, H, N, D, scale);
  if (rc != FA_OK) return rc;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (D != 128) return FA_ERR_UNSUPPORTED;
  const int kind = mask ? mask->kind : FA_MASK_NONE;
  if (smooth && kind == FA_MASK_ADDITIVE) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > 65535) return FA_ERR_SHAPE;   // the prepass grids take B*H as a grid dimension
  if ((int64_t)(N + 256) * D * 2 > (int64_t)UINT32_MAX) return FA_ERR_SHAPE;
  const fa::Int8Layout lay = fa::int8qk_workspace_layout(B, H, N, D, pv16, smooth);
  // one head's compensation table is addressed with 31-bit byte offsets
  if (smooth && (uint64_t)lay.groups * (uint64_t)lay.npad * 4u >= (1ull << 31)) return FA_ERR_SHAPE;
  if (!workspace) return FA_ERR_WORKSPACE;
  if (workspace_bytes < lay.total) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
  fa::MaskArgs m{nullptr, 0, 0, 0, 0};
  if (kind != FA_MASK_NONE) m = fa::MaskArgs{mask->ptr, mask->stride_b, mask->stride_h, mask->stride_q, mask->stride_k};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (log_enabled())
    std::fprintf(stderr, "[fa] %s dtype=%s D=%d mask=%d B=%d H=%d N=%d ws=%zu\n",
                 name, dtype_name(dtype), D, kind, B, H, N, lay.total);
  if (pv16) {
    if (dtype == FA_BF16)
      rc = fa::launch_int8qk_pv16<__bf16>(q, k, v, o, lse, kind, m, B, H, N, scale, workspace, lay, smooth, st);
    else
      rc = fa::launch_int8qk_pv16<_Float16>(q, k, v, o, lse, kind, m, B, H, N, scale, workspace, lay, smooth, st);
  } else {
    if (dtype == FA_BF16)
      rc = fa::launch_int8qk<__bf16>(q, k, v, o, lse, kind, m, B, H, N, scale, workspace, lay, smooth, st);
    else
      rc = fa::launch_int8qk<_Float16>(q, k, v, o, lse, kind, m, B, H, N, scale, workspace, lay, smooth, st);
  }
  if (rc != FA_OK) return rc;
  return record_launch(name);
}
}  // namespace

extern "C" {

FA_API int fa_fwd_int8qk(const void* q, const void* k, const void* v, void* o, float* lse,
                  const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                  fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                  void* hip_stream) {
  return int8qk_common(false, false, q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace, workspace_bytes,
                       hip_stream);
}

FA_API int fa_fwd_int8qk_pv16(const void* q, const void* k, const void* v, void* o, float* lse,
                              const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                              fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
  return int8qk_common(true, false, q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace, workspace_bytes,
                       hip_stream);
}

FA_API int fa_fwd_int8qk_smooth(const void* q, const void* k, const void* v, void* o, float* lse,
                                const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                                fa_dtype_t dtype, int pv16, void* workspace, size_t workspace_bytes,
                                void* hip_stream) {
  if (pv16 != 0 && pv16 != 1) return FA_ERR_ARG;
  return int8qk_common(pv16 != 0, true, q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace,
                       workspace_bytes, hip_stream);
}

FA_API int fa_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o, float* lse, int B, int H, int N, int D, fa_dtype_t dtype,
                    void* hip_stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  const int elt = dtype == FA_F32 ? 4 : 2;
  if ((D * elt) % 16 != 0 || D * elt > 64 * 16) return FA_ERR_UNSUPPORTED;
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse_a, 4) || !aligned(lse_b, 4) || (lse && !aligned(lse, 4))) return FA_ERR_ALIGN;
  const int64_t rows = (int64_t)B * H * N;
  if (rows > (int64_t)1 << 40) return FA_ERR_SHAPE;
  const int cpr = D * elt / 16;
  int lpr = 1;
  while (lpr < cpr) lpr *= 2;
  const int64_t threads = rows * lpr;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return FA_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  switch (dtype) {
    case FA_F32:
      hipLaunchKernelGGL((fa::fa_merge_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, st,
                         static_cast<const float*>(o_a), lse_a, static_cast<const float*>(o_b), lse_b,
                         static_cast<float*>(o), lse, rows, D * elt, cpr, lpr);
      break;
    case FA_F16:
      hipLaunchKernelGGL((fa::fa_merge_kernel<_Float16>), dim3((unsigned)blocks), dim3(256), 0, st,
                         static_cast<const _Float16*>(o_a), lse_a, static_cast<const _Float16*>(o_b), lse_b,
                         static_cast<_Float16*>(o), lse, rows, D * elt, cpr, lpr);
      break;
    default:
      hipLaunchKernelGGL((fa::fa_merge_kernel<__bf16>), dim3((unsigned)blocks), dim3(256), 0, st,
                         static_cast<const __bf16*>(o_a), lse_a, static_cast<const __bf16*>(o_b), lse_b,
                         static_cast<__bf16*>(o), lse, rows, D * elt, cpr, lpr);
      break;
  }
  return record_launch("fa_merge_kernel");
}

FA_API int fa_mfma_probe(int kind, int workgroups, int iters, float* out, void* hip_stream) {
  if (!out) return FA_ERR_NULL;
  if (workgroups <= 0 || iters <= 0) return FA_ERR_SHAPE;
  if (!aligned(out, 4)) return FA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  switch (kind) {
    case fa::kProbeBf16:
      hipLaunchKernelGGL((fa::fa_mfma_probe_kernel<fa::kProbeBf16>), dim3(workgroups), dim3(256), 0, st, out, iters);
      break;
    case fa::kProbeFp8:
      hipLaunchKernelGGL((fa::fa_mfma_probe_kernel<fa::kProbeFp8>), dim3(workgroups), dim3(256), 0, st, out, iters);
      break;
    case fa::kProbeInt8:
      hipLaunchKernelGGL((fa::fa_mfma_probe_kernel<fa::kProbeInt8>), dim3(workgroups), dim3(256), 0, st, out, iters);
      break;
    default:
      return FA_ERR_ARG;
  }
  return record_launch("fa_mfma_probe_kernel");
}

FA_API int fa_cvt_probe(int kind, const float* in, void* out, int64_t n, void* hip_stream) {
  if (!in || !out) return FA_ERR_NULL;
  if (n <= 0 || n % 4 != 0 || n / 4 > (int64_t)INT32_MAX * 256) return FA_ERR_SHAPE;
  if (!aligned(in, 16) || !aligned(out, 8)) return FA_ERR_ALIGN;
  const int64_t quads = n / 4;
  const unsigned blocks = (unsigned)((quads + 255) / 256);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  switch (kind) {
    case fa::kCvtE4m3:
      hipLaunchKernelGGL((fa::fa_cvt_probe_kernel<fa::kCvtE4m3>), dim3(blocks), dim3(256), 0, st, in, out, quads);
      break;
    case fa::kCvtBf16:
      hipLaunchKernelGGL((fa::fa_cvt_probe_kernel<fa::kCvtBf16>), dim3(blocks), dim3(256), 0, st, in, out, quads);
      break;
    case fa::kCvtF16:
      hipLaunchKernelGGL((fa::fa_cvt_probe_kernel<fa::kCvtF16>), dim3(blocks), dim3(256), 0, st, in, out, quads);
      break;
    default:
      return FA_ERR_ARG;
  }
  return record_launch("fa_cvt_probe_kernel");
}

FA_API int fa_int8qk_kv_block(void) { return fa::kInt8Bc; }

FA_API const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H, N or D not positive, or the problem is too large";
    case FA_ERR_UNSUPPORTED: return "dtype / head dimension / mask combination not supported";
    case FA_ERR_ALIGN: return "a pointer is not aligned as required";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_ARG: return "invalid argument";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

FA_API const char* fa_last_hip_error(void) { return g_hip_err; }

FA_API int fa_abi_version(void) { return 4; }

}  // extern "C"
