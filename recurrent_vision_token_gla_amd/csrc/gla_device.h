// Device-side helpers shared by the gfx950 kernels: scan-order index math,
// per-batch direction codes, vector types for the matrix-core builtins, and
// row loads/stores that convert between the storage type and half/float.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kMaxBatchPerLaunch = 1024;

// Control words of the single-pass schedule, at the start of every workspace
// (64 KiB): a header (word 0: sticky error bits) and, per (batch, head) chain
// of a launch, one word per chunk, one per segment and one counter.
constexpr int kCtrlWords = 16384;
constexpr int kCtrlHeader = 64;

// Direction codes of up to kMaxBatchPerLaunch batch elements, 2 bits each,
// passed by value in the kernel arguments (no device copy, graph-safe).
struct DirPack {
  uint32_t w[kMaxBatchPerLaunch / 16];
  __host__ __device__ int get(int b) const { return (w[b >> 4] >> (2 * (b & 15))) & 3; }
};

// Raster index of the token at scan position t (GTR project page, "How GTR
// Works": four scan orders over the patch grid). Left->right is raster
// order; top->bottom walks columns left to right, each top to bottom;
// right->left and bottom->top reverse those two sequences.
// The column walk's t / gh and t % gh: below 2^22 tokens through a float
// reciprocal (the quotient t/gh < 2^22, so the rounded product is within
// 0.75 of it and one step corrects the truncation), else integer division.
__device__ __forceinline__ int scan_to_raster(int t, int T, int gh, int gw, int dir) {
  if (dir & 1) t = T - 1 - t;  // R2L (1) and B2T (3) reverse
  if (dir & 2) {               // T2B (2) and B2T (3)
    int q, r;
    if (T < (1 << 22)) {
      q = (int)((float)t * __builtin_amdgcn_rcpf((float)gh));
      r = t - q * gh;
      if (r < 0) --q, r += gh;
      else if (r >= gh) ++q, r -= gh;
    } else {
      q = t / gh, r = t % gh;
    }
    return r * gw + q;
  }
  return t;
}

// ---- row loads of 8 consecutive elements --------------------------------
__device__ __forceinline__ void load8(const half_t* p, float (&x)[8]) {
  half8 h = *reinterpret_cast<const half8*>(p);
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = (float)h[c];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  floatx4 a = *reinterpret_cast<const floatx4*>(p);
  floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) { x[c] = a[c]; x[c + 4] = b[c]; }
}
__device__ __forceinline__ half8 load8h(const half_t* p) {
  return *reinterpret_cast<const half8*>(p);
}
__device__ __forceinline__ half8 load8h(const float* p) {
  floatx4 a = *reinterpret_cast<const floatx4*>(p);
  floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
  half8 h;
#pragma unroll
  for (int c = 0; c < 4; ++c) { h[c] = (half_t)a[c]; h[c + 4] = (half_t)b[c]; }
  return h;
}

// ---- row stores of 8 consecutive elements from float -----------------------
__device__ __forceinline__ void store8(half_t* p, const float (&x)[8]) {
  half8 h;
#pragma unroll
  for (int c = 0; c < 8; ++c) h[c] = (half_t)x[c];
  *reinterpret_cast<half8*>(p) = h;
}
// Eight consecutive elements of the forward's output o, copied as they are
// (16 or 32 bytes) or converted from float, with the non-temporal hint:
// nothing in the forward reads o again, and on the large grids the output
// and single-pass kernels measured 8-12% faster this way than with
// write-back stores. (Summaries and states, which the next phase reads,
// keep write-back stores.)
__device__ __forceinline__ void out8(half_t* dst, const half_t* src) {
  __builtin_nontemporal_store(*reinterpret_cast<const half8*>(src), reinterpret_cast<half8*>(dst));
}
__device__ __forceinline__ void out8(float* dst, const float* src) {
  __builtin_nontemporal_store(*reinterpret_cast<const floatx4*>(src), reinterpret_cast<floatx4*>(dst));
  __builtin_nontemporal_store(*reinterpret_cast<const floatx4*>(src + 4), reinterpret_cast<floatx4*>(dst + 4));
}
__device__ __forceinline__ void out8(half_t* p, const float (&x)[8]) {
  half8 h;
#pragma unroll
  for (int c = 0; c < 8; ++c) h[c] = (half_t)x[c];
  __builtin_nontemporal_store(h, reinterpret_cast<half8*>(p));
}
__device__ __forceinline__ void out8(float* p, const float (&x)[8]) {
  __builtin_nontemporal_store(floatx4{x[0], x[1], x[2], x[3]}, reinterpret_cast<floatx4*>(p));
  __builtin_nontemporal_store(floatx4{x[4], x[5], x[6], x[7]}, reinterpret_cast<floatx4*>(p + 4));
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  floatx4 a = {x[0], x[1], x[2], x[3]};
  floatx4 b = {x[4], x[5], x[6], x[7]};
  *reinterpret_cast<floatx4*>(p) = a;
  *reinterpret_cast<floatx4*>(p + 4) = b;
}

__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace gla
