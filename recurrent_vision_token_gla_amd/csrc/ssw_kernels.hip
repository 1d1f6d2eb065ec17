// gfx950 kernel of the Spatial SwiGLU channel mixer's fused core.
//
// GTR's channel mixer (ai.info summary of GTR, "Methodology in Plain
// English"; project page, "How GTR Works") inserts a 3x3 depthwise
// convolution, taken on the 2-D patch grid, into the value branch of a
// SwiGLU block. With the two input projections already applied by the caller
// (a = gate branch, u = value branch, both [B][T][F] in raster token order),
// this kernel computes, per token (y, x) and channel c,
//   h[y][x][c] = silu(a[y][x][c]) * (bias[c] + sum_{i,j=0..2} w[c][i][j] u[y+i-1][x+j-1][c])
// with zero padding outside the grid: one read of a and u, one write of h.
//
// A workgroup takes a tile of kTH x kTW tokens and kCF channels. The value
// tile with its one-token halo goes to LDS once; every thread keeps the 3x3
// weights of its 8 channels in registers and produces kItems outputs of 8
// channels (16-byte loads and stores; a token's 64 channels are one
// contiguous 128-byte run).
#include <type_traits>

#include "gla_launch.h"

namespace gla {
namespace {

constexpr int kTH = 8, kTW = 16, kCF = 64;  // tile rows, tile columns, channels
constexpr int kGroups = kCF / 8;            // 8-channel groups per tile
constexpr int kItems = kTH * kTW * kGroups / kThreads;  // outputs per thread
constexpr int kHalo = (kTH + 2) * (kTW + 2);

typedef float float8_t __attribute__((ext_vector_type(8)));  // 8 channels of float

__device__ __forceinline__ float silu(float a) {
  // a * sigmoid(a); exp2 on the transcendental unit, reciprocal of 1 + e^-a
  const float e = __builtin_amdgcn_exp2f(-a * kLog2e);
  return a * __builtin_amdgcn_rcpf(1.f + e);
}

template <typename InT>
__global__ __launch_bounds__(kThreads) void ssw_kernel(const InT* __restrict__ ap,
                                                       const InT* __restrict__ up,
                                                       const float* __restrict__ wp,
                                                       const float* __restrict__ bp,
                                                       InT* __restrict__ hp, int gh, int gw,
                                                       int F, int tiles_w) {
  using StT = InT;  // the value tile is staged in the input precision
  __shared__ __attribute__((aligned(16))) StT sU[kHalo][kCF];
  const int tid = threadIdx.x;
  const int ty0 = (blockIdx.x / tiles_w) * kTH, tx0 = (blockIdx.x % tiles_w) * kTW;
  const int c0 = blockIdx.y * kCF;
  const long bT = (long)blockIdx.z * gh * gw;
  const int ngroups = min(kGroups, (F - c0) / 8);  // F is a multiple of 8

  // -- halo tile of u: (kTH+2) x (kTW+2) tokens x kCF channels, zero outside.
  // A fixed number of clamped, unconditional loads per thread, all issued
  // before the first LDS store waits on one.
  constexpr int kHaloIt = (kHalo * kGroups + kThreads - 1) / kThreads;
  typedef typename std::conditional<sizeof(InT) == 2, half8, float8_t>::type Vec;
  Vec hv[kHaloIt];
#pragma unroll
  for (int k = 0; k < kHaloIt; ++k) {
    const int it = min(tid + kThreads * k, kHalo * kGroups - 1);
    const int p = it / kGroups, g = it % kGroups;
    const int y = ty0 - 1 + p / (kTW + 2), x = tx0 - 1 + p % (kTW + 2);
    const long tok = bT + (long)min(max(y, 0), gh - 1) * gw + min(max(x, 0), gw - 1);
    hv[k] = *reinterpret_cast<const Vec*>(up + tok * F + c0 + 8 * min(g, ngroups - 1));
  }
#pragma unroll
  for (int k = 0; k < kHaloIt; ++k) {
    const int it = tid + kThreads * k;
    if (it < kHalo * kGroups) {
      const int p = it / kGroups, g = it % kGroups;
      const int y = ty0 - 1 + p / (kTW + 2), x = tx0 - 1 + p % (kTW + 2);
      const bool in = y >= 0 && y < gh && x >= 0 && x < gw && g < ngroups;
      *reinterpret_cast<Vec*>(&sU[p][8 * g]) = in ? hv[k] : Vec{};
    }
  }

  // -- this thread's channel group and its weights
  const int g = tid % kGroups;
  const bool gvalid = g < ngroups;
  const int cg = c0 + 8 * min(g, ngroups - 1);
  float w[8][9], bias[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int k = 0; k < 9; ++k) w[c][k] = wp[(long)(cg + c) * 9 + k];
    bias[c] = bp ? bp[cg + c] : 0.f;
  }
  // gate-branch inputs of this thread's outputs (clamped to valid tokens)
  Vec avv[kItems];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int p = tid / kGroups + (kThreads / kGroups) * i;  // token within the tile
    const int y = min(ty0 + p / kTW, gh - 1), x = min(tx0 + p % kTW, gw - 1);
    avv[i] = *reinterpret_cast<const Vec*>(ap + (bT + (long)y * gw + x) * F + cg);
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int p = tid / kGroups + (kThreads / kGroups) * i;
    const int ly = p / kTW, lx = p % kTW;
    const int y = ty0 + ly, x = tx0 + lx;
    float av[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) av[c] = (float)avv[i][c];
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = bias[c];
#pragma unroll
    for (int di = 0; di < 3; ++di) {
#pragma unroll
      for (int dj = 0; dj < 3; ++dj) {
        const StT* s = &sU[(ly + di) * (kTW + 2) + lx + dj][8 * g];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += w[c][3 * di + dj] * (float)s[c];
      }
    }
    if (gvalid && y < gh && x < gw) {
      float out[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) out[c] = silu(av[c]) * acc[c];
      store8(hp + (bT + (long)y * gw + x) * F + cg, out);
    }
  }
}

template <typename InT>
hipError_t ssw_t(const void* a, const void* u, const float* w, const float* bias, void* h, int B,
                 int gh, int gw, int F, hipStream_t s) {
  const int tiles_w = (gw + kTW - 1) / kTW, tiles_h = (gh + kTH - 1) / kTH;
  dim3 grid(tiles_w * tiles_h, (F + kCF - 1) / kCF, B);
  hipLaunchKernelGGL((ssw_kernel<InT>), grid, dim3(kThreads), 0, s, static_cast<const InT*>(a),
                     static_cast<const InT*>(u), w, bias, static_cast<InT*>(h), gh, gw, F,
                     tiles_w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spatial_swiglu(int dtype, const void* a, const void* u, const float* w,
                                 const float* bias, void* h, int B, int gh, int gw, int F,
                                 hipStream_t s) {
  return dtype == 0 ? ssw_t<half_t>(a, u, w, bias, h, B, gh, gw, F, s)
                    : ssw_t<float>(a, u, w, bias, h, B, gh, gw, F, s);
}

}  // namespace gla
