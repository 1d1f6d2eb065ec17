// Device helpers shared by the forward's kernels: exp2, DPP row scans,
// matrix-core wrappers, LDS row reads, the chunk's token rows in scan order,
// and the coherent publish / wait primitives of the single-pass schedule.
#pragma once

#include "gla_device.h"

namespace gla {
namespace tile {

// exp2 on the transcendental unit. Results below 2^-126 flush to zero; every
// factor built with it multiplies a term that is then negligible.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float row_scan16(float x) {
  // inclusive prefix sum over the 16 lanes of each DPP row; a lane whose
  // source lies before the row's start reads 0 (bound_ctrl), which lets each
  // step compile to one add with the shifted operand
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  return x;
}

// x * y as a fused multiply-add with +0: the same value up to the sign of a
// zero result, and, with x converted from a half input, one mixed-precision
// fma instead of a conversion and a product
__device__ __forceinline__ float mulw(float x, float y) { return fmaf(x, y, 0.f); }

// Eight consecutive floats of an LDS row (16-byte aligned) in two reads.
// Per-(sub-block, key dim) factors are fetched this way: eight scalar reads
// under a wave-dependent condition would each be waited for in turn.
__device__ __forceinline__ void lds8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
  x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}

__device__ __forceinline__ floatx4 mfma16x16x16(half4 a, half4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Raster row of scan position tok (-1 past the end of the sequence).
__device__ __forceinline__ int token_row(int tok, int T, int gh, int gw, int dir) {
  return tok < T ? scan_to_raster(tok, T, gh, gw, dir) : -1;
}

// Raster row of every token of the chunk, for the output scatter (tix: the
// thread's index among the chunk's kThreads threads).
template <int C>
__device__ __forceinline__ void chunk_rows(int* sRow, int tok0, int T, int gh, int gw, int dir,
                                           int tix) {
  if (tix < C) sRow[tix] = token_row(tok0 + tix, T, gh, gw, dir);
}

// Token row t of a [B][T][H][D] tensor, this lane's 8*NKS dims
// d = 32*ks + lk + c, in float (zero for padding rows). The loads are
// unconditional (a padding row reads row 0 and is zeroed afterwards): a load
// under a divergent branch would be waited for before the branches rejoin,
// which would serialize every load of the kernel's prologue.
// A padding row's values are zeroed by zero_row afterwards, once every
// prologue load is in flight, and only in a chain's last chunk (a branch
// right after the loads would wait for them).
template <int D, int NKS, typename InT>
__device__ __forceinline__ void load_row(const InT* p, long row, int lk, float* x) {
  const InT* r = p + (row >= 0 ? row : 0) * D + lk;
  float y[NKS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) load8(r + 32 * ks, y[ks]);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int c = 0; c < 8; ++c) x[8 * ks + c] = y[ks][c];
}
// The same row kept as loaded (half rows in their 16-byte vectors), converted
// where each element is consumed: a conversion then folds into the product
// that uses it (v_fma_mix) instead of taking an instruction of its own.
template <typename InT, int NKS> struct RawRow;
template <int NKS> struct RawRow<half_t, NKS> {
  half8 v[NKS];
  __device__ __forceinline__ void load(const half_t* p, long row, int D, int lk) {
    const half_t* r = p + (row >= 0 ? row : 0) * D + lk;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) v[ks] = *reinterpret_cast<const half8*>(r + 32 * ks);
  }
  __device__ __forceinline__ void zero_if(bool pad) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) v[ks] = pad ? half8{} : v[ks];
  }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e / 8][e % 8]; }
};
template <int NKS> struct RawRow<float, NKS> {
  float x[8 * NKS];
  __device__ __forceinline__ void load(const float* p, long row, int D, int lk) {
    load_row<0, NKS>(p + (row >= 0 ? row : 0) * D, 0, lk, x);
  }
  __device__ __forceinline__ void zero_if(bool pad) {
#pragma unroll
    for (int e = 0; e < 8 * NKS; ++e) x[e] = pad ? 0.f : x[e];
  }
  __device__ __forceinline__ float operator[](int e) const { return x[e]; }
};

template <int NEL>
__device__ __forceinline__ void zero_row(bool pad, float* x) {
#pragma unroll
  for (int e = 0; e < NEL; ++e) x[e] = pad ? 0.f : x[e];
}

// A 16x16 block of a row-major half tile in LDS, read through the LDS unit's
// transposing read (ds_read_b64_tr_b16). blk = &tile[R0][c0]; lane
// (i = lane % 16, q = lane / 16) receives rows R0 + GSTEP*q + 0..3 of column
// c0 + i: the matrix-core operand layout of a block whose rows run along the
// contraction (the B operand of the 16x16x16 product, or the A operand of the
// transposed product). The read works within each group of 16 lanes: source
// lane s supplies four consecutive halves (row GSTEP*q + s/4, columns
// 4*(s%4)..+3) and lane i receives element i%4 of source lane 4k + i/4 as its
// k-th value. Rows are 8-byte aligned (STR a multiple of 4); a row stride of
// 16 halves modulo 64 keeps the four rows of a lane group in distinct banks.
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

template <int STR, int GSTEP>
__device__ __forceinline__ half4 ld_tr(const half_t* blk) {
  const int s = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
  const half_t* p = blk + (GSTEP * q + (s >> 2)) * STR + 4 * (s & 3);
  return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)p));
}

// V rows of the chunk (scan positions tok0..tok0+C-1) for sV[token][e]
// (half, zero for padding rows), in two steps: load() issues the 16-byte
// loads into registers (each thread finds its rows' raster positions itself,
// and the loads are unconditional as in RawRow), store() writes them to LDS.
// Work that needs only earlier loads (the decay scan) goes between the two,
// so it does not wait for V. tix: the thread's index among the chunk's
// kThreads threads; a (token, head) row of v holds `pitch` elements, DV of
// them read here.
template <int DV, int C, int VSTR, typename InT>
struct VRows {
  static constexpr int NIT = (C * (DV / 8) + kThreads - 1) / kThreads;
  half8 v8[NIT];
  int rows[NIT];
  __device__ __forceinline__ void load(const InT* vp, int tok0, int T, int gh, int gw, int dir,
                                       long bT, int H, int h, int pitch, int tix) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int u = tix + kThreads * it;
      const int r = (u / (DV / 8)) % C, c8 = (u % (DV / 8)) * 8;
      rows[it] = token_row(tok0 + r, T, gh, gw, dir);
      v8[it] = load8h(vp + ((bT + (rows[it] >= 0 ? rows[it] : 0)) * H + h) * pitch + c8);
    }
  }
  __device__ __forceinline__ void store(int tok0, int T, half_t (*sV)[VSTR], int tix) const {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int u = tix + kThreads * it;
      const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
      if (u < C * (DV / 8)) {
        half8 x = v8[it];
        if (tok0 + C > T && rows[it] < 0) x = half8{};  // padding row (last chunk only)
        *reinterpret_cast<half8*>(&sV[r][c8]) = x;
      }
    }
  }
};

__device__ __forceinline__ void load_f8(const float* p, float (&a)[8]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  const float4 y = *reinterpret_cast<const float4*>(p + 4);
  a[0] = x.x, a[1] = x.y, a[2] = x.z, a[3] = x.w;
  a[4] = y.x, a[5] = y.y, a[6] = y.z, a[7] = y.w;
}

__device__ __forceinline__ void store_f8(float* p, const float (&a)[8]) {
  *reinterpret_cast<float4*>(p) = float4{a[0], a[1], a[2], a[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{a[4], a[5], a[6], a[7]};
}

// ---- power-of-two scales that keep half tiles in range ----------------------
// A state row (summary U, boundary state S, look-back aggregate) is stored in
// half divided by a power of two sigma >= 1: sigma = 1 while the row's largest
// magnitude m stays below 2^14, else the power of two that brings m into
// [2^13, 2^14). So the stored values stay far inside the half range and the
// row keeps float's upper range. Zero and non-finite m give sigma = 1.
constexpr float kRowRange = 16384.f;  // 2^14
__device__ __forceinline__ float row_scale(float m) {
  const int eb = (int)((__float_as_uint(m) >> 23) & 0xffu);  // m >= 0: biased exponent
  const int e = eb - 140;  // m < 2^(eb-126), so m / 2^e < 2^14
  return (e <= 0 || eb == 255) ? 1.f : __uint_as_float((unsigned)(e + 127) << 23);
}
// LDS offsets rounded up to 16 bytes
constexpr int lds_round(int x) { return (x + 15) & ~15; }

// A value the caller knows to be equal on every lane, made a scalar so that
// branches on it are scalar branches (the compiler cannot see the equality).
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// 1 / sigma, exact (sigma is a power of two between 1 and 2^114)
__device__ __forceinline__ float inv_scale(float sigma) {
  return __uint_as_float(((254u << 23) - __float_as_uint(sigma)) & 0x7f800000u);
}
// The exponent e >= 0 of row_scale(m) = 2^e, without a branch (non-finite m
// gives a large scale; such rows are non-finite anyway).
__device__ __forceinline__ int row_scale_exp(float m) {
  return max((int)((__float_as_uint(m) >> 23) & 0xffu) - 140, 0);
}

// Eight floats to half with the packed round-to-nearest-even conversion.
typedef float floatx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ half8 cvt8(const float (&x)[8]) {
  const floatx8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, half8);
}
__device__ __forceinline__ half4 cvt4(const floatx4& x) { return __builtin_convertvector(x, half4); }

// Largest value over the aligned group of LANES consecutive lanes the caller
// belongs to (every lane of the group active): DPP lane permutations within
// a row of 16 (quad swaps, then the half-row mirror), shuffles beyond.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float m) {
  return fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), CTRL, 0xf,
                                                              0xf, false)));
}
template <int LANES>
__device__ __forceinline__ float group_max(float m) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64, "");
  m = dpp_max<0xB1>(m);                       // quad_perm [1,0,3,2]: lane ^ 1
  m = dpp_max<0x4E>(m);                       // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LANES >= 8) m = dpp_max<0x141>(m);   // row_half_mirror: the other quad
  if constexpr (LANES >= 16) m = dpp_max<0x140>(m);  // row_mirror: the other half-row
  if constexpr (LANES >= 32) m = fmaxf(m, __shfl_xor(m, 16));
  if constexpr (LANES >= 64) m = fmaxf(m, __shfl_xor(m, 32));
  return m;
}

// A (decay, row scale) pair published as one 8-byte device-coherent access.
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {
  const unsigned long long v =
      (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32))};
}

template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float x, float fill) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// ===========================================================================
// Single-pass schedule: control words at the start of the workspace.
//   word 0            sticky error bits (kErrSpin: a bounded wait ran out)
//   per chain c (one (batch, head) of a launch), kCtrlHeader + c*(N+nseg+1):
//     [0, N)          chunk n has published U_n and a_n
//     [N, N+nseg)     segment s has published its aggregate
//     [N+nseg]        chunks of the chain that have finished reading
// All of them are zero between calls: the last chunk of a chain to finish
// reading clears the chain's words, so a workspace zeroed once stays valid.
// ===========================================================================
constexpr unsigned kErrSpin = 1u;
constexpr long kSpinLimit = 1L << 21;  // polls of one wait (seconds, far above any real wait)

// Data one workgroup publishes for others in the same kernel (summaries, their
// decays, segment aggregates) is written and read only with device-scope
// atomic accesses (relaxed, 8 or 4 bytes). Those are coherent across the
// XCDs' L2 caches by themselves, so publishing needs no L2 write-back and
// reading no L2 invalidation, which would cost every workgroup on the XCD:
//   publisher: coherent stores; each wave waits for their completion and
//              counts itself in LDS; the last one stores the flag.
//   reader:    one wave polls the flags; barrier; coherent loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Tiles of half (U, segment aggregates) move as 16-byte buffer accesses with
// the device-scope cache policy (sc1): the coherence of the atomics below,
// one instruction per 16 bytes (two interleaved 8-byte atomics would write
// every 32-byte sector twice). The resource covers one chain's array;
// accesses outside it read zero and write nothing.
constexpr int kCohDevice = 16;  // cache-policy bits: sc1
constexpr unsigned kBufWord3 = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const half_t* base, long halves) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(base), 0, (int)(2 * halves), kBufWord3);
}
__device__ __forceinline__ void st_coh(__amdgpu_buffer_rsrc_t r, int half_off, half8 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, 2 * half_off, 0, kCohDevice);
}
__device__ __forceinline__ half8 ld_coh(__amdgpu_buffer_rsrc_t r, int half_off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * half_off, 0, kCohDevice));
}

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Marks loaded registers as read on every path. A load whose result a
// branch skips stays outstanding past the join for the compiler's wait
// insertion, so the next write of that register would wait for all memory
// operations issued since (stores included); here the wait comes where the
// value is consumed anyway.
__device__ __forceinline__ void consume(const half8& u, const float& a) {
  asm volatile("" ::"v"(u), "v"(a));
}

// Lane i of the calling wave watches flags[i], i < count <= 64. Returns once
// every watched flag is set, or when the poll budget runs out (recorded in
// *err). The caller then passes a workgroup barrier before reading.
__device__ __forceinline__ void wave_wait_flags(const unsigned* flags, int count, unsigned* err) {
  const int lane = threadIdx.x & 63;
  if (count <= 0) return;
  for (long it = 0;; ++it) {
    bool ok = true;
    if (lane < count)
      ok = __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (__all(ok)) break;
    if (it >= kSpinLimit) {
      if (lane == 0) atomicOr(err, kErrSpin);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Called once by every wave of a chunk's kThreads threads after it has
// issued its coherent stores of one publication: the wave waits for their
// completion and counts itself in *count (LDS, zero beforehand); the last
// wave to arrive sets the flag to value. No barrier, so a wave that arrives
// early goes on.
__device__ __forceinline__ void publish_wave(unsigned* flag, unsigned* count, unsigned value = 1u) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0 && atomicAdd(count, 1u) == kThreads / 64 - 1)
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Status words of a chain's runs for the decoupled look-back between runs:
// 0 nothing yet, kStAgg the run's own aggregate is published, kStInc its
// inclusive state (everything before it folded in) is.
constexpr unsigned kStAgg = 1u, kStInc = 2u;

// Called by one wave for run `run` > 0 of a chain whose status words are
// st[0..]: waits until some predecessor p has kStInc with every run between
// p and `run` at least kStAgg, or every predecessor down to the chain's start
// is at least kStAgg. Returns the number of aggregates to fold in (the runs
// run-1 down to p+1, or all of them) and sets *from_start when the chain's
// start (the initial state) takes the place of an inclusive state. Windows
// of 64 predecessors, one lane each; every wait is bounded (running out sets
// the sticky error bit in *err and returns with results invalid).
__device__ __forceinline__ int lookback_runs(const unsigned* st, int run, unsigned* err,
                                            int* from_start) {
  const int lane = threadIdx.x & 63;
  for (int j0 = 0;; j0 += 64) {
    const int cnt = min(64, run - j0);  // predecessors run-1-j0-lane, lane < cnt
    for (long it = 0;; ++it) {
      unsigned v = 0u;
      if (lane < cnt)
        v = __hip_atomic_load(st + (run - 1 - j0 - lane), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long inc = __ballot(lane < cnt && v == kStInc);
      const unsigned long long none = __ballot(lane < cnt && v == 0u);
      if (inc) {
        const int jl = __builtin_ctzll(inc);
        if ((none & ((1ull << jl) - 1ull)) == 0ull) {
          *from_start = 0;
          return j0 + jl;
        }
      } else if (none == 0ull) {
        if (j0 + cnt == run) {  // every predecessor aggregated: start from the initial state
          *from_start = 1;
          return run;
        }
        break;  // all aggregated: the next window
      }
      if (it >= kSpinLimit) {
        if (lane == 0) atomicOr(err, kErrSpin);
        *from_start = 1;
        return j0 + cnt;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

}  // namespace tile
}  // namespace gla
