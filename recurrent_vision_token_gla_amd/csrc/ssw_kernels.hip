// gfx950 kernel of the Spatial SwiGLU channel mixer's fused core.
//
// GTR's channel mixer (ai.info summary of GTR, "Methodology in Plain
// English"; project page, "How GTR Works") is a SwiGLU whose non-gated input
// path first passes through a per-channel 3x3 spatial filter over the patch
// grid. With the two input projections already applied by the caller
// (a = gate branch, u = value branch, both [B][T][F] in raster token order),
// this kernel computes, per token (y, x) and channel c,
//   h[y][x][c] = silu(a[y][x][c]) * (bias[c] + sum_{i,j=0..2} w[c][i][j] u[y+i-1][x+j-1][c])
// with zero padding outside the grid: one read of a and u, one write of h.
//
// A workgroup takes a tile of kTH x kTW tokens and kCF channels. The value
// tile with its one-token halo goes to LDS once; every thread keeps the 3x3
// weights of its 8 channels in registers and produces kItems outputs of 8
// channels (16-byte loads and stores; a token's 64 channels are one
// contiguous 128-byte run). The persistent form further down is used whenever
// ten grid rows of the value tensor fit a 32-bit buffer offset; the
// grid-per-tile kernel that comes first covers wider grids.
#include <cstdint>
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
      out8(hp + (bT + (long)y * gw + x) * F + cg, out);
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent, double-buffered form. A grid of about three workgroups per CU
// walks the (batch, channel block, tile) units with a stride. While a unit
// is computed from one LDS buffer, the next unit's halo tile streams into the
// other with buffer loads that write LDS directly (lane l of a load lands 16 *
// l bytes past the wave's base; a position outside the grid or the channels
// gets an offset past its buffer's end and reads zero, which is the zero
// padding), and its gate inputs into registers. The 3x3 weights and biases
// (fp32) also come by direct loads, into one LDS buffer that is refilled once
// every thread has copied the current unit's into registers. Each unit then
// costs about the longer of its loads and its arithmetic, and no round of
// workgroups runs partly empty.
// ---------------------------------------------------------------------------
template <typename InT>
struct SswPipe {
  static constexpr int kUPT = kCF * (int)sizeof(InT) / 16;  // 16-byte units per halo token
  static constexpr int kUnits = kHalo * kUPT;               // of the halo tile
  static constexpr int kFull = kUnits / kThreads;           // rounds every wave loads
  static constexpr int kRemWaves = (kUnits - kFull * kThreads + 63) / 64;  // waves of the last round
  static constexpr int kHaloBytes = (kFull * kThreads + kRemWaves * 64) * 16;
  static constexpr int kWBytes = 3 * 64 * 16;  // 576 fp32 weights: 144 units, three waves' loads
  static constexpr int kBBytes = 64 * 16;      // 64 fp32 biases: 16 units, one wave's load
  static constexpr int kLdsBytes = 2 * kHaloBytes + kWBytes + kBBytes;
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename InT>
__global__ __launch_bounds__(kThreads, 3) void ssw_persistent(
    const InT* __restrict__ ap, const InT* __restrict__ up, const float* __restrict__ wp,
    const float* __restrict__ bp, InT* __restrict__ hp, int gh, int gw, int F, int tiles_w,
    int ntiles, int ncb, int nunits) {
  using P = SswPipe<InT>;
  using StT = InT;
  typedef typename std::conditional<sizeof(InT) == 2, half8, float8_t>::type Vec;
  __shared__ __attribute__((aligned(16))) char smem[P::kLdsBytes];
  char* sW = smem + 2 * P::kHaloBytes;  // weights [64][9], then biases [64]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = tid % kGroups;
  const long T = (long)gh * gw;
  const int wnum = F * 9 * 4, bnum = bp ? F * 4 : 0;  // bytes of weights and biases
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(wp), 0, wnum, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(bp), 0, bnum, 0x00020000);

  struct Unit {
    int b, cb, ty0, tx0;
  };
  // units numbered channel block fastest: the workgroups running at one time
  // cover whole token rows of the [T][F] tensors
  auto unit = [&](int id) {
    const int cb = id % ncb, r = id / ncb, tile = r % ntiles;
    return Unit{r / ntiles, cb, (tile / tiles_w) * kTH, (tile % tiles_w) * kTW};
  };
  // halo tile of unit U into buffer buf: every wave issues kFull loads, the
  // first kRemWaves one more
  // the resource starts at the unit's first halo row (y = ty0 - 1, which may
  // lie before the tensor: only positions inside the grid are read) and spans
  // kTH + 2 grid rows, so offsets stay 32-bit for any number of rows
  const unsigned nbytes = (unsigned)((long)(kTH + 2) * gw * F * (long)sizeof(InT));
  auto load_halo = [&](const Unit& U, int buf) {
    const uintptr_t rbase = reinterpret_cast<uintptr_t>(up) +
                            (uintptr_t)(((long)U.b * T + (long)(U.ty0 - 1) * gw) * F * (long)sizeof(InT));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(rbase), 0, (int)nbytes, 0x00020000);
    char* base = smem + buf * P::kHaloBytes + 1024 * wave;
    const int c0 = U.cb * kCF;
#pragma unroll
    for (int k = 0; k <= P::kFull; ++k) {
      if (k == P::kFull && wave >= P::kRemWaves) break;
      const int it = tid + kThreads * k;
      const int p = it / P::kUPT, e = (it % P::kUPT) * (16 / (int)sizeof(StT));  // token, channel
      const int py = p / (kTW + 2), y = U.ty0 - 1 + py, x = U.tx0 - 1 + p % (kTW + 2);
      const bool in = it < P::kUnits && y >= 0 && y < gh && x >= 0 && x < gw && c0 + e < F;
      const unsigned off = in ? (unsigned)((((long)py * gw + x) * F + c0 + e) * sizeof(InT)) : nbytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(base + kThreads * 16 * k), 16, off, 0, 0, 0);
    }
  };
  // weights and biases of channel block cb: waves 0-2 load the 144 weight
  // units, wave 3 the 16 bias units (one load per wave)
  auto load_wb = [&](int cb) {
    const int j = 64 * wave + lane;
    if (wave < 3) {
      const unsigned off = j < 144 ? (unsigned)(cb * kCF * 9 * 4 + 16 * j) : (unsigned)wnum;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(sW + 1024 * wave), 16, off, 0, 0, 0);
    } else {
      const unsigned off = lane < 16 ? (unsigned)(cb * kCF * 4 + 16 * lane) : (unsigned)bnum;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(sW + P::kWBytes), 16, off, 0, 0, 0);
    }
  };
  // gate-branch input of output i of this thread (clamped to a valid token)
  auto load_a = [&](const Unit& U, int i) {
    const int cg = min(U.cb * kCF + 8 * g, F - 8);
    const int p = tid / kGroups + (kThreads / kGroups) * i;
    const int y = min(U.ty0 + p / kTW, gh - 1), x = min(U.tx0 + p % kTW, gw - 1);
    return *reinterpret_cast<const Vec*>(ap + ((long)U.b * T + (long)y * gw + x) * F + cg);
  };

  int id = blockIdx.x;
  if (id >= nunits) return;
  Unit cur = unit(id);
  Vec av[kItems];  // gate inputs of the unit being computed; refilled item by item for the next
  load_halo(cur, 0);
  load_wb(cur.cb);
#pragma unroll
  for (int i = 0; i < kItems; ++i) av[i] = load_a(cur, i);
  for (int k = 0;; ++k) {
    const int nid = id + gridDim.x;
    const bool more = nid < nunits;
    const Unit nxt = unit(more ? nid : id);
    if (more) {
      load_halo(nxt, (k + 1) & 1);
      // everything issued before the next unit's halo (this unit's halo,
      // weights, biases and gate inputs, the previous unit's stores) is
      // complete once no more than that halo's loads are outstanding
      if (wave < P::kRemWaves) wait_vm<P::kFull + 1>();
      else wait_vm<P::kFull>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    // -- this thread's channel group: weights and biases into registers
    const int c0 = cur.cb * kCF;
    const bool gvalid = c0 + 8 * g < F;
    float w[8][9], bias[8];
    {
      const float* sw = reinterpret_cast<const float*>(sW) + (8 * g) * 9;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int q = 0; q < 9; ++q) w[c][q] = sw[9 * c + q];
      const float* sb = reinterpret_cast<const float*>(sW + P::kWBytes) + 8 * g;
#pragma unroll
      for (int c = 0; c < 8; ++c) bias[c] = sb[c];
    }
    __syncthreads();  // every thread has its weights: the buffer takes the next unit's
    if (more) load_wb(nxt.cb);
    // -- outputs
    const StT(*sU)[kCF] = reinterpret_cast<const StT(*)[kCF]>(smem + (k & 1) * P::kHaloBytes);
    const long bT = (long)cur.b * T;
    const int cg = c0 + 8 * g;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int p = tid / kGroups + (kThreads / kGroups) * i;
      const int ly = p / kTW, lx = p % kTW;
      const int y = cur.ty0 + ly, x = cur.tx0 + lx;
      float acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = bias[c];
#pragma unroll
      for (int di = 0; di < 3; ++di) {
#pragma unroll
        for (int dj = 0; dj < 3; ++dj) {
          const StT* sv = &sU[(ly + di) * (kTW + 2) + lx + dj][8 * g];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] += w[c][3 * di + dj] * (float)sv[c];
        }
      }
      if (gvalid && y < gh && x < gw) {
        float out[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) out[c] = silu((float)av[i][c]) * acc[c];
        out8(hp + (bT + (long)y * gw + x) * F + cg, out);
      }
      if (more) av[i] = load_a(nxt, i);
    }
    if (!more) break;
    __syncthreads();  // this buffer is free for the unit after next
    id = nid;
    cur = nxt;
  }
}

template <typename InT>
int ssw_blocks_per_cu() {
  static int cached[64];  // per device; 0 = not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cached[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ssw_persistent<InT>, kThreads, 0) != hipSuccess || nb < 1)
      nb = 1;
    cached[dev] = nb;
  }
  return cached[dev];
}

template <typename InT>
hipError_t ssw_t(const void* a, const void* u, const float* w, const float* bias, void* h, int B,
                 int gh, int gw, int F, hipStream_t s) {
  const int tiles_w = (gw + kTW - 1) / kTW, tiles_h = (gh + kTH - 1) / kTH;
  const int ncb = (F + kCF - 1) / kCF;
  // the persistent form while kTH + 2 grid rows of the value tensor stay below
  // 2^31 bytes (32-bit buffer offsets, plus the out-of-range offset)
  if ((long)(kTH + 2) * gw * F * (long)sizeof(InT) < (1L << 31) && (long)F * 9 * 4 < (1L << 31)) {
    const long nunits = (long)B * ncb * tiles_w * tiles_h;
    if (nunits < (1L << 31)) {
      int dev = 0, ncu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        ncu = 1;
      const long cap = (long)ncu * ssw_blocks_per_cu<InT>();
      const int grid = (int)(nunits < cap ? nunits : cap);
      hipLaunchKernelGGL((ssw_persistent<InT>), dim3(grid), dim3(kThreads), 0, s,
                         static_cast<const InT*>(a), static_cast<const InT*>(u), w, bias,
                         static_cast<InT*>(h), gh, gw, F, tiles_w, tiles_w * tiles_h, ncb,
                         (int)nunits);
      return hipGetLastError();
    }
  }
  dim3 grid(tiles_w * tiles_h, ncb, B);
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
