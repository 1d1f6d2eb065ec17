// gfx950 kernels of the chunkwise key-only GLA forward.
//
// Schedule (GTR project page, "A Kernel That Makes Recurrence Fast"; ai.info
// summary of GTR, "Methodology in Plain English"): per-chunk summaries in
// parallel over the chunk x head grid, a light scan of the chunk-boundary
// states along the chunk axis, then every chunk's outputs in parallel with the
// causal intra-chunk tile held on chip (LDS) and the boundary-state readout
// fused in. All three phases read their tokens through the scan-order index
// math, so no permuted copy of any tensor is ever made.
//
// Notation inside a chunk of C tokens (local index i), per key dim d, with
// g2 = gk * log2(e) so that every exponential is a base-2 exp2:
//   b_i = sum_{r<=i} g2_r                 inclusive cumulative log2-decay
//   B   = b_{C-1}                          (padding tokens have g2 = 0)
// Every factor fed to a half-precision matrix product is <= 1 in magnitude
// (times |q| or |k|), so strong decay cannot overflow it:
//   summary : K^[j] = k_j * 2^(B - b_j)
//   readout : Q^[i] = q_i * 2^(b_i)
//   off-diagonal 16x16 sub-blocks (I > J) of the score tile:
//       Q~[i] = q_i 2^(b_i - beta_I),  K~[j] = k_j 2^(e_J - b_j),
//       m_IJ  = 2^(beta_I - e_J)
//     with beta_I = b at the token before sub-block I and e_J = b at the
//     last token of sub-block J; A_IJ = (Q~_I * m_IJ) K~_J^T.
//   diagonal sub-blocks are exact for any gk <= 0: running products of the
//     per-token decays 2^(g2), never a ratio of two exponentials.
#include "gla_launch.h"

namespace gla {
namespace {


// ---------------------------------------------------------------------------
// Helpers shared by the phase kernels.
// ---------------------------------------------------------------------------
// exp2 on the transcendental unit. Results below 2^-126 flush to zero; every
// factor built with it multiplies a term that is then negligible.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float row_scan16(float x) {
  // inclusive prefix sum over the 16 lanes of each DPP row
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
  return x;
}

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

// Raster row of every token of the chunk (-1 past the end of the sequence).
template <int C>
__device__ __forceinline__ void chunk_rows(int* sRow, int tok0, int T, int gh, int gw, int dir) {
  const int tid = threadIdx.x;
  const int L = min(C, T - tok0);
  if (tid < C) sRow[tid] = tid < L ? scan_to_raster(tok0 + tid, T, gh, gw, dir) : -1;
}

// Token row t of a [B][T][H][D] tensor, this lane's 8*NKS dims
// d = 32*ks + lk + c, in float (zero for padding rows). The loads are
// unconditional (a padding row reads row 0 and is zeroed afterwards): a load
// under a divergent branch would be waited for before the branches rejoin,
// which would serialize every load of the kernel's prologue.
template <int D, int NKS, typename InT>
__device__ __forceinline__ void load_row(const InT* p, long row, int lk, float* x) {
  const bool valid = row >= 0;
  const InT* r = p + (valid ? row : 0) * D + lk;
  float y[NKS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) load8(r + 32 * ks, y[ks]);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int c = 0; c < 8; ++c) x[8 * ks + c] = valid ? y[ks][c] : 0.f;
}

// V rows of the chunk, transposed into sVt[e][token] (half); loads
// unconditional as in load_row.
template <int DV, int C, int VSTR, typename InT>
__device__ __forceinline__ void load_vt(const InT* vp, const int* sRow, long bT, int H, int h,
                                        half_t (*sVt)[VSTR]) {
  constexpr int NIT = (C * (DV / 8) + kThreads - 1) / kThreads;
  half8 v8[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int u = threadIdx.x + kThreads * it;
    const int r = (u / (DV / 8)) % C, c8 = (u % (DV / 8)) * 8;
    const int row = sRow[r] >= 0 ? sRow[r] : 0;
    v8[it] = load8h(vp + ((bT + row) * H + h) * DV + c8);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int u = threadIdx.x + kThreads * it;
    const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
    if (u < C * (DV / 8)) {
      const bool valid = sRow[r] >= 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) sVt[c8 + c][r] = valid ? v8[it][c] : (half_t)0.f;
    }
  }
}

// ===========================================================================
// Phase 1: chunk summaries. One workgroup per (chunk n, head h, batch b).
//   U[d][e] = sum_j K^[j][d] V[j][e],     K^[j] = k_j 2^(B - b_j)  (<= |k|)
//   a[d]      = 2^(B[d])
// Wave w owns the 16 tokens of sub-block w, one token per lane row, and
// takes its cumulative decay with a DPP row scan plus the totals of the
// earlier sub-blocks. K^ goes to LDS transposed (token-contiguous per key
// dim), V likewise, so both operands of the token contraction are 8-byte
// LDS reads; U is produced (as U^T) in 16x16 blocks on the matrix cores,
// staged through LDS as rows of key dims and stored as half [dk][dv].
// ===========================================================================
template <int DK, int DV, int C, typename InT>
__global__ __launch_bounds__(kThreads, 7) void summary_kernel(
    const InT* __restrict__ kp, const InT* __restrict__ vp, const InT* __restrict__ gp,
    half_t* __restrict__ Uws, float* __restrict__ Aws, int T, int H, int N, int gh, int gw,
    DirPack dirs) {
  constexpr int NB = C / 16, NKS = DK / 32, NEL = 8 * NKS, NE = DV / 16, ND = DK / 16;
  constexpr int VSTR = C + 8;    // halves, token-contiguous rows
  constexpr int USTR = DV + 8;   // halves, staging rows of U (one row per key dim)
  // the U staging tile reuses K^T's LDS once the products have read it
  constexpr int KU_BYTES = (VSTR > USTR ? VSTR : USTR) * DK * 2;
  __shared__ __attribute__((aligned(16))) half_t sVt[DV][VSTR];
  __shared__ __attribute__((aligned(16))) char sKU[KU_BYTES];
  __shared__ __attribute__((aligned(16))) float sTot[NB][DK];
  __shared__ __attribute__((aligned(16))) float sAft[NB][DK];  // totals of sub-blocks I..NB-1
  __shared__ int sRow[C];
  half_t (*sKh)[VSTR] = reinterpret_cast<half_t (*)[VSTR]>(sKU);
  half_t (*sU)[USTR] = reinterpret_cast<half_t (*)[USTR]>(sKU);

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = 8 * lq;
  chunk_rows<C>(sRow, n * C, T, gh, gw, dirs.get(b));
  __syncthreads();

  const bool owner = wave < NB;
  const int I = wave, t = 16 * I + lr;
  float kf[NEL], sc[NEL];
  {
    const int rr = owner ? sRow[t] : -1;
    const long row = rr >= 0 ? ((long)b * T + rr) * H + h : -1;
    load_row<DK, NKS>(kp, row, lk, kf);
    load_row<DK, NKS>(gp, row, lk, sc);
  }
  load_vt<DV, C, VSTR>(vp, sRow, (long)b * T, H, h, sVt);
  if (owner) {
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(sc[e] * kLog2e);
    if (lr == 15) {
#pragma unroll
      for (int e = 0; e < NEL; ++e) sTot[I][32 * (e / 8) + lk + (e % 8)] = sc[e];
    }
  }
  __syncthreads();

  const long bhn = ((long)b * H + h) * N + n;
  if (tid < NB * DK) {
    const int I2 = tid / DK, d = tid % DK;
    float aft = 0.f;
    for (int J = I2; J < NB; ++J) aft += sTot[J][d];
    sAft[I2][d] = aft;
    if (I2 == 0) Aws[bhn * DK + d] = fexp2(aft);  // a = 2^B
  }
  __syncthreads();
  if (owner) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float aft[8];
      lds8(&sAft[I][32 * ks + lk], aft);
#pragma unroll
      for (int c = 0; c < 8; ++c)  // B - b_t: the decay of the later tokens
        sKh[32 * ks + lk + c][t] = (half_t)(kf[8 * ks + c] * fexp2(aft[c] - sc[8 * ks + c]));
    }
  }
  __syncthreads();

  constexpr int NBLK = NE * ND, BPW = (NBLK + 3) / 4;  // output blocks per wave
  floatx4 acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + 4 * i;
    acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (blk < NBLK) {
      const int E = blk / ND, D = blk % ND;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        const half4 a = *reinterpret_cast<const half4*>(&sVt[16 * E + lr][16 * J + 4 * lq]);
        const half4 bb = *reinterpret_cast<const half4*>(&sKh[16 * D + lr][16 * J + 4 * lq]);
        acc[i] = mfma16x16x16(a, bb, acc[i]);
      }
    }
  }
  __syncthreads();  // K^T is no longer read
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + 4 * i;
    if (blk < NBLK) {
      const int E = blk / ND, D = blk % ND;
      half4 h;
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = (half_t)acc[i][r];
      *reinterpret_cast<half4*>(&sU[16 * D + lr][16 * E + 4 * lq]) = h;
    }
  }
  __syncthreads();
  half_t* Ub = Uws + bhn * (long)(DV * DK);
  for (int u = tid; u < DK * (DV / 8); u += kThreads) {
    const int d = u / (DV / 8), e8 = (u % (DV / 8)) * 8;
    *reinterpret_cast<half8*>(Ub + d * DV + e8) = *reinterpret_cast<const half8*>(&sU[d][e8]);
  }
}

// ===========================================================================
// Phase 2: boundary-state scan. Every state element (d, e) of one (batch,
// head) is its own first-order recurrence over the chunks,
//   S_0 = given or 0,  S_{n+1}[d][e] = a_n[d] * S_n[d][e] + U_n[d][e],
// and the step (a, U) composes associatively:
//   (a1, U1) then (a2, U2) = (a2 a1, a2 U1 + U2).
// So the chunk axis is cut into 16 segments, one per lane of a DPP row:
// each lane folds its segment into one (a, U) pair, a 4-step row scan gives
// every segment the composition of all earlier ones, and each lane then
// replays its segment from the exact entering state, storing S_n (half,
// [dk][dv]) for the output phase. A lane covers 8 consecutive value columns
// of one key dim, so it needs a single decay per chunk; the four rows of a
// wave take four neighbouring element groups, so each chunk's loads and
// stores are 64-byte runs. The state after the last chunk (the composition
// over all 16 segments, applied to S_0) is optionally written in fp32.
// ===========================================================================
constexpr int kScanSegs = 16;  // segments per chain: the lanes of a DPP row

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

template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float x, float fill) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// R: chunks per segment kept in registers (2, 4 or 8, the segment length
// rounded up, so that the clamped loads of a short segment are not repeated)
template <int kScanRegs>
__global__ __launch_bounds__(kThreads) void scan_kernel(const half_t* __restrict__ Uws,
                                                        const float* __restrict__ Aws,
                                                        half_t* __restrict__ Sws,
                                                        const float* __restrict__ s0,
                                                        float* __restrict__ sfin, int H, int N,
                                                        int DK, int DV, int L) {
  const long bh = (long)blockIdx.z * H + blockIdx.y;
  const int seg = threadIdx.x & (kScanSegs - 1);
  const int x8 = 8 * (blockIdx.x * (kThreads / kScanSegs) + (threadIdx.x >> 4));
  const int d = x8 / DV;
  const long DKDV = (long)DK * DV;
  const half_t* U = Uws + bh * N * DKDV + x8;
  const float* A = Aws + bh * N * DK + d;
  half_t* S = Sws + bh * N * DKDV + x8;
  const int n0 = min(seg * L, N), n1 = min(n0 + L, N);

  // -- fold this segment into (ag, ug); the chunks of one register block stay cached
  float ag = 1.f, ug[8];
  half8 uc[kScanRegs];
  float ac[kScanRegs];
#pragma unroll
  for (int c = 0; c < 8; ++c) ug[c] = 0.f;
  for (int nb = n0; nb < n1; nb += kScanRegs) {
    // clamped, unconditional loads (all in flight together); chunks past
    // the segment's end are read but not used
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) {
      const long m = min(nb + i, n1 - 1);
      uc[i] = *reinterpret_cast<const half8*>(U + m * DKDV);
      ac[i] = A[m * DK];
    }
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) {
      if (nb + i < n1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) ug[c] = ac[i] * ug[c] + (float)uc[i][c];
        ag *= ac[i];
      }
    }
  }
  // -- inclusive composition over the segments of this row, then shift by one
#define GLA_SCAN_STEP(CTRL)                                              \
  {                                                                      \
    const float ap = dpp_row_shr<CTRL>(ag, 1.f);                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) ug[c] =                \
        ag * dpp_row_shr<CTRL>(ug[c], 0.f) + ug[c];                      \
    ag *= ap;                                                            \
  }
  GLA_SCAN_STEP(0x111)
  GLA_SCAN_STEP(0x112)
  GLA_SCAN_STEP(0x114)
  GLA_SCAN_STEP(0x118)
#undef GLA_SCAN_STEP
  float st0[8], s[8];
  if (s0) {
    load_f8(s0 + bh * DKDV + x8, st0);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) st0[c] = 0.f;
  }
  const float ae = dpp_row_shr<0x111>(ag, 1.f);
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = ae * st0[c] + dpp_row_shr<0x111>(ug[c], 0.f);
  if (sfin && seg == kScanSegs - 1) {
    float f[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) f[c] = ag * st0[c] + ug[c];
    store_f8(sfin + bh * DKDV + x8, f);
  }
  // -- replay the segment from its entering state; a segment longer than one
  // register block reads its chunks again (the registers hold the last block)
  const bool cached = n1 - n0 <= kScanRegs;
  for (int nb = n0; nb < n1; nb += kScanRegs) {
    if (!cached) {
#pragma unroll
      for (int i = 0; i < kScanRegs; ++i) {
        const long m = min(nb + i, n1 - 1);
        uc[i] = *reinterpret_cast<const half8*>(U + m * DKDV);
        ac[i] = A[m * DK];
      }
    }
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) {
      if (nb + i < n1) {
        store8(S + (long)(nb + i) * DKDV, s);
#pragma unroll
        for (int c = 0; c < 8; ++c) s[c] = ac[i] * s[c] + (float)uc[i][c];
      }
    }
  }
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
//   publisher: coherent stores; each wave waits for their completion;
//              barrier; one flag store.
//   reader:    one wave polls the flags; barrier; coherent loads.
typedef unsigned long u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void st_dev(half_t* p, half8 v) {
  const u64x2 w = __builtin_bit_cast(u64x2, v);
  unsigned long* q = reinterpret_cast<unsigned long*>(p);
  __hip_atomic_store(q, w.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, w.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ half8 ld_dev(const half_t* p) {
  const unsigned long* q = reinterpret_cast<const unsigned long*>(p);
  u64x2 w;
  w.x = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  w.y = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(half8, w);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Every wave waits until its coherent stores have completed, then one flag
// is set. Must be reached by the whole workgroup.
__device__ __forceinline__ void publish(unsigned* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ===========================================================================
// Chunk outputs. One workgroup per (chunk n, head h, batch b).
//   O = A V + Q^ S_n,   A = causal decayed score tile
//
// Wave w owns query sub-block I = w (tokens 16I..16I+15). A lane holds one
// token row (lr = lane % 16) and 8*DK/32 key dims d = 32*ks + 8*(lane/16) + c,
// which is exactly the operand layout of the 16x16x32 matrix-core product, so
// the per-element factors are computed in registers and fed to the matrix
// cores directly. Within a sub-block, with s_i = sum of g2 over its tokens up
// to i and tot = s_15 (all log2):
//   Q~ = q 2^(s_i)   K~ = k 2^(tot - s_i)   Q^ = Q~ 2^(beta_I)
// Score sub-blocks are produced transposed (A^T = K Q^T), so each lane ends
// up holding A[i = lr][j = 4*(lane/16) + r], the operand layout of the 16x16x16
// product A V: the score tile stays in registers, never round-tripping LDS.
//   off-diagonal J < I: A_IJ = (Q~_I * m_IJ) K~_J^T, m_IJ = 2^(beta_I - e_J)
//   diagonal:           A_II = Q' K'^T with Q' = q 2^(s_i - s_7),
//                       K' = k 2^(s_7 - s_j): one reference at the 8th token.
// The diagonal block uses half operands when no key dim decays by more than
// 2^8 over a sub-block, fp32 operands up to 2^120, and beyond that (checked
// per tile) sums every entry directly from 2^(s_i - s_j).
//
// kFused = false: phase 3 of three; S_n comes from the boundary scan.
// kFused = true: the whole forward in one pass (the chunk summary, the
// boundary state and the outputs). Workgroups run in chain-major order, so a
// chunk only ever waits on chunks of lower index, which were dispatched
// earlier. Each chunk
//   1. computes its summary U_n and decay a_n and publishes them;
//   2. computes its intra-chunk part A V while its predecessors publish;
//   3. takes the state it enters, in two levels over segments of G chunks:
//        S_n = X + W (.) P,  X = sum_{s0 <= m < n} (prod_{m<j<n} a_j) (.) U_m,
//        W = prod_{s0 <= j < n} a_j,  P = state entering the segment
//      where P composes the aggregates (prod a, sum of decayed U) that the
//      last chunk of each earlier segment publishes (and the initial state);
//   4. adds the readout Q^ S_n and stores the outputs.
// ===========================================================================
template <int DK, int DV, int C, typename InT, bool kFused>
__global__ __launch_bounds__(kThreads, 4) void chunk_kernel(
    const InT* __restrict__ qp, const InT* __restrict__ kp, const InT* __restrict__ vp,
    const InT* __restrict__ gp, InT* __restrict__ op, half_t* __restrict__ Uws,
    float* __restrict__ Aws, half_t* __restrict__ Sws, float* __restrict__ GAws,
    unsigned* __restrict__ ctrl, const float* __restrict__ s0, float* __restrict__ sfin, int T,
    int H, int N, int G, int nseg, int gh, int gw, DirPack dirs) {
  constexpr int NB = C / 16, NKS = DK / 32, NEL = 8 * NKS, NE = DV / 16, ND = DK / 16;
  constexpr int NPAIR = NB * (NB - 1) / 2;
  constexpr int DKDV = DK * DV;
  constexpr int KSTR = DK + 8;  // halves, rows of K~ and S^T
  constexpr int VSTR = C + 8;   // halves, rows of V^T and K^T
  constexpr int USTR = DV + 8;  // halves, rows of the U staging tile
  constexpr int OSTR = DV + 8;  // rows of the output staging tile
  constexpr int NGR = (DKDV / 8 + kThreads - 1) / kThreads;  // state groups of 8 per thread
  constexpr int LB = 4;  // predecessors per batch of look-back loads
  constexpr float kHalfRange = 8.f, kF32Range = 120.f;  // log2 decay per sub-block
  // K~ is dead once the score blocks are built; the output tile reuses it
  constexpr int KO_BYTES = (C * KSTR * 2 > C * OSTR * (int)sizeof(InT)) ? C * KSTR * 2
                                                                        : C * OSTR * (int)sizeof(InT);
  // one region in turn holds K^T, the U staging tile and S^T (only S^T unfused)
  constexpr int X0 = DV * KSTR * 2, X1 = kFused ? DK * VSTR * 2 : 0, X2 = kFused ? DK * USTR * 2 : 0;
  constexpr int X_BYTES = X0 > X1 ? (X0 > X2 ? X0 : X2) : (X1 > X2 ? X1 : X2);
  __shared__ __attribute__((aligned(16))) char sKO[KO_BYTES];
  __shared__ __attribute__((aligned(16))) half_t sVt[DV][VSTR];
  __shared__ __attribute__((aligned(16))) char sX[X_BYTES];
  __shared__ __attribute__((aligned(16))) float sTot[NB][DK], sS7[NB][DK];
  __shared__ __attribute__((aligned(16))) float sEb[NB][DK], sR1[NB][DK], sR2[NB][DK];
  __shared__ __attribute__((aligned(16))) float sM[NPAIR > 0 ? NPAIR : 1][DK];
  __shared__ __attribute__((aligned(16))) float sF[kFused ? NB : 1][DK];  // K^ = K~ * sF
  __shared__ float sAn[kFused ? DK : 1];
  __shared__ int sRow[C];
  __shared__ int sTier;
  __shared__ unsigned sDone;
  half_t (*sKt)[KSTR] = reinterpret_cast<half_t (*)[KSTR]>(sKO);
  InT (*sO)[OSTR] = reinterpret_cast<InT (*)[OSTR]>(sKO);
  half_t (*sS)[KSTR] = reinterpret_cast<half_t (*)[KSTR]>(sX);
  half_t (*sKh)[VSTR] = reinterpret_cast<half_t (*)[VSTR]>(sX);
  half_t (*sU)[USTR] = reinterpret_cast<half_t (*)[USTR]>(sX);

  int n, h, b;
  if constexpr (kFused) {
    const int bh = blockIdx.x / N;
    n = blockIdx.x - bh * N, h = bh % H, b = bh / H;
  } else {
    n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  }
  const long bh = (long)b * H + h, bhn = bh * N + n;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = 8 * lq;
  chunk_rows<C>(sRow, n * C, T, gh, gw, dirs.get(b));
  if (tid == 0) sTier = 0;
  __syncthreads();

  // -- this wave's token rows of q, k, gk in the operand layout (waves past
  // the last sub-block load a padding row too: no branch around the loads)
  const bool owner = wave < NB;
  const int I = wave, t = 16 * I + lr;
  float qf[NEL], kf[NEL], sc[NEL];
  {
    const int rr = owner ? sRow[t] : -1;
    const long row = rr >= 0 ? ((long)b * T + rr) * H + h : -1;
    load_row<DK, NKS>(qp, row, lk, qf);
    load_row<DK, NKS>(kp, row, lk, kf);
    load_row<DK, NKS>(gp, row, lk, sc);
  }
  // -- the entering state (stored [dk][dv], staged transposed as sS[e][d];
  // three-phase schedule only) and the chunk's V^T, through LDS; every load
  // is issued before the first LDS write that waits on one
  constexpr int NSIT = kFused ? 1 : (DKDV / 8 + kThreads - 1) / kThreads;
  half8 h8[NSIT];
  if constexpr (!kFused) {
    const half_t* Sb = Sws + bhn * (long)DKDV;
#pragma unroll
    for (int it = 0; it < NSIT; ++it) h8[it] = load8h(Sb + 8 * ((tid + kThreads * it) % (DKDV / 8)));
  }
  load_vt<DV, C, VSTR>(vp, sRow, (long)b * T, H, h, sVt);
  if constexpr (!kFused) {
#pragma unroll
    for (int it = 0; it < NSIT; ++it) {
      const int u = tid + kThreads * it;
      if (u < DKDV / 8) {
        const int d = u / (DV / 8), e8 = (u % (DV / 8)) * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) sS[e8 + c][d] = h8[it][c];
      }
    }
  }

  // -- in-sub-block inclusive cumsum along tokens (DPP row scan)
  if (owner) {
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(sc[e] * kLog2e);
    if (lr == 15 || lr == 7) {
#pragma unroll
      for (int e = 0; e < NEL; ++e) {
        const int d = 32 * (e / 8) + lk + (e % 8);
        if (lr == 15) sTot[I][d] = sc[e];
        else sS7[I][d] = sc[e];
      }
    }
  }
  __syncthreads();

  // -- per (sub-block, key dim) factors, one key dim per thread
  if (tid < NB * DK) {
    const int I2 = tid / DK, d = tid % DK;
    float beta = 0.f;
    for (int J = 0; J < I2; ++J) beta += sTot[J][d];
    const float tot = sTot[I2][d], s7 = sS7[I2][d];
    sEb[I2][d] = fexp2(beta);
    sR1[I2][d] = fexp2(-s7);
    sR2[I2][d] = fexp2(s7 - tot);
    float acc = 0.f;  // log2 of m_{I2,J} for J = I2-1, I2-2, ...
    for (int J = I2 - 1; J >= 0; --J) {
      sM[I2 * (I2 - 1) / 2 + J][d] = fexp2(acc);
      acc += sTot[J][d];
    }
    const float range = -tot;
    if (!(range <= kF32Range)) atomicMax(&sTier, 2);
    else if (!(range <= kHalfRange)) atomicMax(&sTier, 1);
    if constexpr (kFused) {
      float after = 0.f;  // totals of the later sub-blocks
      for (int J = I2 + 1; J < NB; ++J) after += sTot[J][d];
      sF[I2][d] = fexp2(after);
      if (I2 == NB - 1) sAn[d] = fexp2(beta + tot);  // a_n = 2^(chunk total)
    }
  }
  __syncthreads();
  // -- per-element factors; K~ goes to LDS for the other sub-blocks, and in
  // one pass K^ = K~ 2^(totals of the later sub-blocks), transposed, for U
  float qt[NEL], kt[NEL];
  if (owner) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float tt[8], ff[8];
      lds8(&sTot[I][32 * ks + lk], tt);
      if constexpr (kFused) lds8(&sF[I][32 * ks + lk], ff);
      half8 k8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = 8 * ks + c, d = 32 * ks + lk + c;
        qt[e] = qf[e] * fexp2(sc[e]);
        kt[e] = kf[e] * fexp2(tt[c] - sc[e]);
        k8[c] = (half_t)kt[e];
        if constexpr (kFused) sKh[d][t] = (half_t)(kt[e] * ff[c]);
      }
      *reinterpret_cast<half8*>(&sKt[t][32 * ks + lk]) = k8;
    }
  }
  __syncthreads();

  unsigned* cw = nullptr;  // this chain's control words
  if constexpr (kFused) {
    cw = ctrl + kCtrlHeader + bh * (long)(N + nseg + 1);
    // -- U_n^T = V^T K^ in 16x16 blocks, staged as rows of key dims, published
    constexpr int NBLK = NE * ND, BPW = (NBLK + 3) / 4;
    floatx4 uacc[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      uacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (blk < NBLK) {
        const int E = blk / ND, D = blk % ND;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          const half4 a = *reinterpret_cast<const half4*>(&sVt[16 * E + lr][16 * J + 4 * lq]);
          const half4 bb = *reinterpret_cast<const half4*>(&sKh[16 * D + lr][16 * J + 4 * lq]);
          uacc[i] = mfma16x16x16(a, bb, uacc[i]);
        }
      }
    }
    __syncthreads();  // K^T is no longer read: the region becomes the U staging tile
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      if (blk < NBLK) {
        const int E = blk / ND, D = blk % ND;
        half4 hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (half_t)uacc[i][r];
        *reinterpret_cast<half4*>(&sU[16 * D + lr][16 * E + 4 * lq]) = hv;
      }
    }
    __syncthreads();
    // wave 0 alone stores and flags U_n and a_n, so that the other waves go
    // on to their score blocks without waiting for the stores to complete
    if (wave == 0) {
      for (int x8 = 8 * lane; x8 < DKDV; x8 += 8 * 64)
        st_dev(Uws + bhn * DKDV + x8, *reinterpret_cast<const half8*>(&sU[x8 / DV][x8 % DV]));
      for (int d = lane; d < DK; d += 64) st_dev(Aws + bhn * DK + d, sAn[d]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(cw + n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  half4 A[NB];
  half8 qh[NKS];
  if (owner) {
    const int tier = sTier;
    // -- diagonal sub-block, transposed: acc[r] = A[i = lr][j = 4*lq + r]
    floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
    if (tier == 0) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float r1[8], r2[8];
        lds8(&sR1[I][32 * ks + lk], r1);
        lds8(&sR2[I][32 * ks + lk], r2);
        half8 qa, ka;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          qa[c] = (half_t)(qt[8 * ks + c] * r1[c]);
          ka[c] = (half_t)(kt[8 * ks + c] * r2[c]);
        }
        dacc = mfma16x16x32(ka, qa, dacc);
      }
    } else if (tier == 1) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float r1[8], r2[8];
        lds8(&sR1[I][32 * ks + lk], r1);
        lds8(&sR2[I][32 * ks + lk], r2);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[8 * ks + c] * r2[c], qt[8 * ks + c] * r1[c],
                                                      dacc, 0, 0, 0);
      }
    } else {
      // every entry directly: A_ij = sum_d q_i k_j 2^(s_i - s_j)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < NEL; ++e) {
          const float kj = __shfl(kf[e], (lane & 48) | j);
          const float sj = __shfl(sc[e], (lane & 48) | j);
          part += qf[e] * kj * fexp2(sc[e] - sj);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if ((j >> 2) == lq) dacc[j & 3] = part;
      }
    }
    half4 adiag;
#pragma unroll
    for (int r = 0; r < 4; ++r) adiag[r] = (half_t)((4 * lq + r <= lr) ? dacc[r] : 0.f);
#pragma unroll
    for (int J = 0; J < NB; ++J)
      if (J == I) A[J] = adiag;
    // -- off-diagonal sub-blocks J < I
#pragma unroll
    for (int J = 0; J < NB - 1; ++J) {
      if (J < I) {
        const int pr = I * (I - 1) / 2 + J;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float mm[8];
          lds8(&sM[pr][32 * ks + lk], mm);
          half8 qm;
#pragma unroll
          for (int c = 0; c < 8; ++c) qm[c] = (half_t)(qt[8 * ks + c] * mm[c]);
          const half8 ka = *reinterpret_cast<const half8*>(&sKt[16 * J + lr][32 * ks + lk]);
          acc = mfma16x16x32(ka, qm, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) A[J][r] = (half_t)acc[r];
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float eb[8];
      lds8(&sEb[I][32 * ks + lk], eb);
#pragma unroll
      for (int c = 0; c < 8; ++c) qh[ks][c] = (half_t)(qt[8 * ks + c] * eb[c]);
    }
  }

  if constexpr (!kFused) {
    __syncthreads();  // K~ is no longer read: its LDS becomes the output tile
    // -- O_I = Q^_I S + sum_{J<=I} A_IJ V_J
    if (owner) {
#pragma unroll
      for (int E = 0; E < NE; ++E) {
        // one accumulation chain of a single product shape (16x16x16) per value
        // block: the readout contracts four key dims per lane group per step
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb =
                *reinterpret_cast<const half4*>(&sS[16 * E + lr][32 * ks + lk + 4 * hh]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            acc = mfma16x16x16(qa, sb, acc);
          }
        }
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = *reinterpret_cast<const half4*>(&sVt[16 * E + lr][16 * J + 4 * lq]);
            acc = mfma16x16x16(A[J], vb, acc);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[16 * I + 4 * lq + r][16 * E + lr] = (InT)acc[r];
      }
    }
  } else {
    // -- intra-chunk part first: O_I = sum_{J<=I} A_IJ V_J
    floatx4 oacc[NE];
#pragma unroll
    for (int E = 0; E < NE; ++E) {
      oacc[E] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (owner) {
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = *reinterpret_cast<const half4*>(&sVt[16 * E + lr][16 * J + 4 * lq]);
            oacc[E] = mfma16x16x16(A[J], vb, oacc[E]);
          }
        }
      }
    }
    // -- the entering state, in-segment part: X and W
    const int seg = n / G, n0 = seg * G, nlast = min(n0 + G, N) - 1;
    if (wave == 0) wave_wait_flags(cw + n0, n - n0, ctrl);
    __syncthreads();
    float xs[NGR][8], wv[NGR];
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      wv[g] = 1.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) xs[g][c] = 0.f;
    }
    // all groups' loads of a batch of predecessors go out together
    for (int m = n - 1; m >= n0; m -= LB) {
      half8 u[NGR][LB];
      float a[NGR][LB];
#pragma unroll
      for (int g = 0; g < NGR; ++g) {  // clamped, unconditional loads
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const long mj = m - j >= n0 ? m - j : n0;
          u[g][j] = ld_dev(Uws + (bh * N + mj) * DKDV + x8);
          a[g][j] = ld_dev(Aws + (bh * N + mj) * DK + x8 / DV);
        }
      }
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          if (x8 < DKDV && m - j >= n0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) xs[g][c] += wv[g] * (float)u[g][j][c];
            wv[g] *= a[g][j];
          }
        }
      }
    }
    // -- the last chunk of a segment publishes the segment's aggregate
    if (n == nlast && seg < nseg - 1) {
      const long gs = bh * nseg + seg;
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
        if (x8 < DKDV) {
          half8 ag;
          const half8 un = ld_dev(Uws + bhn * DKDV + x8);  // this chunk's own U_n
#pragma unroll
          for (int c = 0; c < 8; ++c) ag[c] = (half_t)(sAn[d] * xs[g][c] + (float)un[c]);
          st_dev(Sws + gs * DKDV + x8, ag);
        }
      }
      // the segment's decay: the weight the look-back accumulated, times a_n
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
        if (x8 < DKDV && x8 % DV == 0) st_dev(GAws + gs * DK + d, wv[g] * sAn[d]);
      }
      publish(cw + N + seg);
    }
    // -- the state entering the segment, from the earlier segments' aggregates
    if (wave == 0) wave_wait_flags(cw + N, seg, ctrl);
    __syncthreads();
    float pv[NGR][8], w2[NGR];
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      w2[g] = 1.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) pv[g][c] = 0.f;
    }
    for (int s2 = seg - 1; s2 >= 0; s2 -= LB) {
      half8 u[NGR][LB];
      float a[NGR][LB];
#pragma unroll
      for (int g = 0; g < NGR; ++g) {  // clamped, unconditional loads
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const long sj = s2 - j >= 0 ? s2 - j : 0;
          u[g][j] = ld_dev(Sws + (bh * nseg + sj) * DKDV + x8);
          a[g][j] = ld_dev(GAws + (bh * nseg + sj) * DK + x8 / DV);
        }
      }
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          if (x8 < DKDV && s2 - j >= 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) pv[g][c] += w2[g] * (float)u[g][j][c];
            w2[g] *= a[g][j];
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
      if (x8 < DKDV) {
        if (s0) {
          float z[8];
          load_f8(s0 + bh * DKDV + x8, z);
#pragma unroll
          for (int c = 0; c < 8; ++c) pv[g][c] += w2[g] * z[c];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[g][c] += wv[g] * pv[g][c];  // S_n
        if (sfin && n == N - 1) {
          float f[8];
          const half8 un = ld_dev(Uws + bhn * DKDV + x8);
#pragma unroll
          for (int c = 0; c < 8; ++c) f[c] = sAn[d] * xs[g][c] + (float)un[c];
          store_f8(sfin + bh * DKDV + x8, f);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) sS[x8 % DV + c][d] = (half_t)xs[g][c];
      }
    }
    // -- every read of published data is done: count it; the last clears the chain
    __syncthreads();
    if (tid == 0) sDone = atomicAdd(cw + N + nseg, 1u);
    __syncthreads();
    if (sDone == (unsigned)(N - 1))
      for (int i = tid; i < N + nseg + 1; i += kThreads) cw[i] = 0u;
    // -- readout, on the same accumulation chains: O_I += Q^_I S_n
    if (owner) {
#pragma unroll
      for (int E = 0; E < NE; ++E) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb =
                *reinterpret_cast<const half4*>(&sS[16 * E + lr][32 * ks + lk + 4 * hh]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            oacc[E] = mfma16x16x16(qa, sb, oacc[E]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[16 * I + 4 * lq + r][16 * E + lr] = (InT)oacc[E][r];
      }
    }
  }
  __syncthreads();

  // -- scatter rows back to their raster positions
  for (int u = tid; u < C * (DV / 8); u += kThreads) {
    const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
    if (sRow[r] >= 0) {
      float x[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = (float)sO[r][c8 + c];
      store8(op + (((long)b * T + sRow[r]) * H + h) * DV + c8, x);
    }
  }
}

__global__ void scan_perm_kernel(int32_t* perm, int T, int gh, int gw, int dir) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) perm[t] = scan_to_raster(t, T, gh, gw, dir);
}

// ---------------------------------------------------------------------------
template <int DK, int DV, int C, typename InT>
hipError_t summaries_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* k,
                       const void* v, const void* gk, char* ws, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  dim3 grid(p.N, p.H, nb);
  hipLaunchKernelGGL((summary_kernel<DK, DV, C, InT>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(k) + tok * DK, static_cast<const InT*>(v) + tok * DV,
                     static_cast<const InT*>(gk) + tok * DK,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhn * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_a) + bhn * DK, p.T, p.H, p.N, p.gh,
                     p.gw, dirs);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename InT>
hipError_t outputs_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                     const void* k, const void* v, const void* gk, void* o, const char* ws,
                     hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  dim3 grid(p.N, p.H, nb);
  hipLaunchKernelGGL((chunk_kernel<DK, DV, C, InT, false>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     static_cast<InT*>(o) + tok * DV, nullptr, nullptr,
                     const_cast<half_t*>(reinterpret_cast<const half_t*>(ws + w.off_S)) +
                         bhn * DK * DV,
                     nullptr, nullptr, nullptr, nullptr, p.T, p.H, p.N, 1, 1, p.gh, p.gw, dirs);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename InT>
hipError_t onepass_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                     const void* k, const void* v, const void* gk, void* o, char* ws,
                     const float* s0, float* sfin, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const Segments sg = onepass_segments(p.N);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  const long bhs = (long)b0 * p.H * sg.nseg;
  const long st = (long)b0 * p.H * DK * DV;
  // chain-major: every chunk of one (batch, head) before the next chain
  dim3 grid((unsigned)((long)nb * p.H * p.N));
  hipLaunchKernelGGL((chunk_kernel<DK, DV, C, InT, true>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     static_cast<InT*>(o) + tok * DV,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhn * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_a) + bhn * DK,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhs * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_g) + bhs * DK,
                     reinterpret_cast<unsigned*>(ws), s0 ? s0 + st : nullptr,
                     sfin ? sfin + st : nullptr, p.T, p.H, p.N, sg.G, sg.nseg, p.gh, p.gw, dirs);
  return hipGetLastError();
}

__global__ void ctrl_clear_kernel(unsigned* ctrl) {
  for (int i = threadIdx.x; i < kCtrlWords; i += blockDim.x) ctrl[i] = 0u;
}

#define GLA_DISPATCH(FN, ...)                                                          \
  do {                                                                                 \
    const bool f16 = p.dtype == 0;                                                     \
    const int key = (p.dk == 64) * 100 + (p.dv == 64) * 10 + (p.chunk / 16);           \
    switch (key) {                                                                     \
      case 1: return f16 ? FN<32, 32, 16, half_t>(__VA_ARGS__) : FN<32, 32, 16, float>(__VA_ARGS__); \
      case 2: return f16 ? FN<32, 32, 32, half_t>(__VA_ARGS__) : FN<32, 32, 32, float>(__VA_ARGS__); \
      case 4: return f16 ? FN<32, 32, 64, half_t>(__VA_ARGS__) : FN<32, 32, 64, float>(__VA_ARGS__); \
      case 11: return f16 ? FN<32, 64, 16, half_t>(__VA_ARGS__) : FN<32, 64, 16, float>(__VA_ARGS__); \
      case 12: return f16 ? FN<32, 64, 32, half_t>(__VA_ARGS__) : FN<32, 64, 32, float>(__VA_ARGS__); \
      case 14: return f16 ? FN<32, 64, 64, half_t>(__VA_ARGS__) : FN<32, 64, 64, float>(__VA_ARGS__); \
      case 101: return f16 ? FN<64, 32, 16, half_t>(__VA_ARGS__) : FN<64, 32, 16, float>(__VA_ARGS__); \
      case 102: return f16 ? FN<64, 32, 32, half_t>(__VA_ARGS__) : FN<64, 32, 32, float>(__VA_ARGS__); \
      case 104: return f16 ? FN<64, 32, 64, half_t>(__VA_ARGS__) : FN<64, 32, 64, float>(__VA_ARGS__); \
      case 111: return f16 ? FN<64, 64, 16, half_t>(__VA_ARGS__) : FN<64, 64, 16, float>(__VA_ARGS__); \
      case 112: return f16 ? FN<64, 64, 32, half_t>(__VA_ARGS__) : FN<64, 64, 32, float>(__VA_ARGS__); \
      case 114: return f16 ? FN<64, 64, 64, half_t>(__VA_ARGS__) : FN<64, 64, 64, float>(__VA_ARGS__); \
      default: return hipErrorInvalidValue;                                            \
    }                                                                                  \
  } while (0)

}  // namespace

WsLayout workspace_layout(const Problem& p) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t units = (size_t)p.B * p.H * p.N;
  WsLayout w;
  w.off_U = (size_t)kCtrlWords * sizeof(unsigned);
  w.off_a = w.off_U + up(units * p.dk * p.dv * sizeof(half_t));
  w.off_S = w.off_a + up(units * p.dk * sizeof(float));
  w.off_g = w.off_S + up(units * p.dk * p.dv * sizeof(half_t));
  w.total = w.off_g + up(units * p.dk * sizeof(float));
  return w;
}

Segments onepass_segments(int N) {
  int G = 1;
  while (G * G < N) ++G;
  return Segments{G, (N + G - 1) / G};
}

bool onepass_fits(const Problem& p, int nb) {
  const Segments sg = onepass_segments(p.N);
  if (sg.G > 64 || sg.nseg > 64) return false;  // one wave watches every flag it waits on
  const long words = kCtrlHeader + (long)nb * p.H * (p.N + sg.nseg + 1);
  return words <= kCtrlWords && (long)nb * p.H * p.N <= 0x7fffffffL;
}

hipError_t launch_summaries(const Problem& p, int b0, int nb, const DirPack& dirs,
                            const void* k, const void* v, const void* gk, char* ws,
                            hipStream_t s) {
  GLA_DISPATCH(summaries_t, p, b0, nb, dirs, k, v, gk, ws, s);
}

hipError_t launch_scan(const Problem& p, int b0, int nb, char* ws, const float* s0,
                       float* sfin, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const long bhn = (long)b0 * p.H * p.N;
  const long dkdv = (long)p.dk * p.dv;
  const long st = (long)b0 * p.H * dkdv;
  const int L = (p.N + kScanSegs - 1) / kScanSegs;
  // 16 element groups of 8 per workgroup; dk*dv is a multiple of 1024
  dim3 grid((unsigned)(dkdv / (8 * (kThreads / kScanSegs))), p.H, nb);
  auto kernel = L <= 2 ? scan_kernel<2> : L <= 4 ? scan_kernel<4> : scan_kernel<8>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s,
                     reinterpret_cast<const half_t*>(ws + w.off_U) + bhn * dkdv,
                     reinterpret_cast<const float*>(ws + w.off_a) + bhn * p.dk,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhn * dkdv,
                     s0 ? s0 + st : nullptr, sfin ? sfin + st : nullptr, p.H, p.N, p.dk, p.dv,
                     L);
  return hipGetLastError();
}

hipError_t launch_outputs(const Problem& p, int b0, int nb, const DirPack& dirs,
                          const void* q, const void* k, const void* v, const void* gk,
                          void* o, const char* ws, hipStream_t s) {
  GLA_DISPATCH(outputs_t, p, b0, nb, dirs, q, k, v, gk, o, ws, s);
}

hipError_t launch_onepass(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                          const void* k, const void* v, const void* gk, void* o, char* ws,
                          const float* s0, float* sfin, hipStream_t s) {
  GLA_DISPATCH(onepass_t, p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
}

hipError_t launch_ctrl_clear(char* ws, hipStream_t s) {
  hipLaunchKernelGGL(ctrl_clear_kernel, dim3(1), dim3(1024), 0, s, reinterpret_cast<unsigned*>(ws));
  return hipGetLastError();
}

hipError_t launch_scan_perm(int32_t* perm, int gh, int gw, int dir, hipStream_t s) {
  const int T = gh * gw;
  hipLaunchKernelGGL(scan_perm_kernel, dim3((T + 255) / 256), dim3(256), 0, s, perm, T, gh, gw,
                     dir);
  return hipGetLastError();
}

}  // namespace gla
