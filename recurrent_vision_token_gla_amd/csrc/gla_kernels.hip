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

template <int DK, int DV, int C>
struct Geo {
  static constexpr int CP = C < 32 ? 32 : C;  // token extent padded to MFMA depth
  static constexpr int KSTR = DK + 8;         // row stride (halves), [C][DK] tiles
  static constexpr int VSTR = DV + 8;         // row stride (halves), [C][DV] tiles
  static constexpr int TSTR = CP + 8;         // row stride (halves), [D][CP] tiles
  static constexpr int NSEG = kThreads / DK;  // token segments of the cumsum
  static constexpr int SEGLEN = C / NSEG;     // tokens per segment
  static constexpr int NB = C / 16;           // 16-token sub-blocks per chunk
  static constexpr int NPAIR = NB * (NB - 1) / 2;
  static_assert(SEGLEN >= 1 && 16 % SEGLEN == 0, "segment must tile a sub-block");
  static_assert(C % 16 == 0 && DK % 32 == 0 && DV % 16 == 0, "shape");
};

// ===========================================================================
// Phase 1: chunk summaries. One workgroup per (chunk n, head h, batch b).
//   U^T[e][d] = sum_j V[j][e] * K^[j][d]   (stored transposed, row e)
//   a[d]      = 2^(B[d])
// ===========================================================================
template <int DK, int DV, int C, typename InT>
__global__ __launch_bounds__(kThreads) void summary_kernel(
    const InT* __restrict__ kp, const InT* __restrict__ vp, const InT* __restrict__ gp,
    float* __restrict__ Uws, float* __restrict__ Aws, int T, int H, int N, int gh, int gw,
    DirPack dirs) {
  using G = Geo<DK, DV, C>;
  __shared__ __attribute__((aligned(16))) float sG[C][DK];
  __shared__ __attribute__((aligned(16))) half_t sK[C][G::KSTR];
  __shared__ __attribute__((aligned(16))) half_t sV[C][G::VSTR];
  __shared__ __attribute__((aligned(16))) half_t sKt[DK][G::TSTR];
  __shared__ __attribute__((aligned(16))) half_t sVt[DV][G::TSTR];
  __shared__ float sTot[G::NSEG][DK];
  __shared__ int sRow[C];

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int tok0 = n * C;
  const int L = min(C, T - tok0);
  if (tid < C) sRow[tid] = tid < L ? scan_to_raster(tok0 + tid, T, gh, gw, dirs.get(b)) : -1;
  __syncthreads();

  // -- load k, gk (rows of dk) and v (rows of dv); padding rows are zero
  for (int u = tid; u < C * (DK / 8); u += kThreads) {
    const int r = u / (DK / 8), c8 = (u % (DK / 8)) * 8;
    float g8[8];
    half8 k8;
    if (sRow[r] >= 0) {
      const long row = ((long)b * T + sRow[r]) * H + h;
      load8(gp + row * DK + c8, g8);
      k8 = load8h(kp + row * DK + c8);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) { g8[c] = 0.f; k8[c] = (half_t)0.f; }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sG[r][c8 + c] = g8[c] * kLog2e;
    *reinterpret_cast<half8*>(&sK[r][c8]) = k8;
  }
  for (int u = tid; u < C * (DV / 8); u += kThreads) {
    const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
    half8 v8;
    if (sRow[r] >= 0) {
      const long row = ((long)b * T + sRow[r]) * H + h;
      v8 = load8h(vp + row * DV + c8);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v8[c] = (half_t)0.f;
    }
    *reinterpret_cast<half8*>(&sV[r][c8]) = v8;
  }
  __syncthreads();

  // -- inclusive cumsum along tokens, one key dim per thread-column
  const int d = tid % DK, seg = tid / DK;
  float p[G::SEGLEN];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < G::SEGLEN; ++i) {
    run += sG[seg * G::SEGLEN + i][d];
    p[i] = run;
  }
  sTot[seg][d] = run;
  __syncthreads();
  float off = 0.f, tot = 0.f;
#pragma unroll
  for (int s = 0; s < G::NSEG; ++s) {
    const float x = sTot[s][d];
    if (s < seg) off += x;
    tot += x;
  }
  // K^ transposed into [d][token]
#pragma unroll
  for (int i = 0; i < G::SEGLEN; ++i) {
    const int j = seg * G::SEGLEN + i;
    sKt[d][j] = (half_t)((float)sK[j][d] * exp2f(tot - (off + p[i])));
  }
  const long bhn = ((long)b * H + h) * N + n;
  if (seg == 0) Aws[bhn * DK + d] = exp2f(tot);
  // V transposed into [e][token]
  for (int u = tid; u < DV * (C / 8); u += kThreads) {
    const int e = u % DV, j8 = (u / DV) * 8;
    half8 x;
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = sV[j8 + c][e];
    *reinterpret_cast<half8*>(&sVt[e][j8]) = x;
  }
  if constexpr (G::CP > C) {
    for (int u = tid; u < (DK + DV) * (G::CP - C); u += kThreads) {
      const int row = u / (G::CP - C), col = C + u % (G::CP - C);
      if (row < DK) sKt[row][col] = (half_t)0.f;
      else sVt[row - DK][col] = (half_t)0.f;
    }
  }
  __syncthreads();

  // -- U^T = V^T K^ on the matrix cores, 16x16 output blocks, K = tokens
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = 8 * (lane >> 4);
  constexpr int NBD = DK / 16, NBLK = (DV / 16) * NBD;
  float* Ub = Uws + bhn * (long)(DV * DK);
  for (int blk = wave; blk < NBLK; blk += 4) {
    const int E = blk / NBD, D = blk % NBD;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < G::CP / 32; ++ks) {
      const half8 a = *reinterpret_cast<const half8*>(&sVt[16 * E + lr][32 * ks + lk]);
      const half8 bb = *reinterpret_cast<const half8*>(&sKt[16 * D + lr][32 * ks + lk]);
      acc = mfma16x16x32(a, bb, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) Ub[(16 * E + 4 * (lane >> 4) + r) * DK + 16 * D + lr] = acc[r];
  }
}

// ===========================================================================
// Phase 2: boundary-state scan. One thread per state element (e, d) of one
// (batch, head); a wave covers 64 consecutive d of one value column e, so
// every load and store is a coalesced row segment. Serial over chunks:
//   S_0 = 0,  S_{n+1}[e][d] = a_n[d] * S_n[e][d] + U_n^T[e][d]
// The state entering each chunk is stored (half, transposed [e][d]).
// ===========================================================================
__global__ __launch_bounds__(kThreads) void scan_kernel(const float* __restrict__ Uws,
                                                        const float* __restrict__ Aws,
                                                        half_t* __restrict__ Sws, int N,
                                                        int DK, int DKDV) {
  const long bh = blockIdx.y;
  const int x = blockIdx.x * kThreads + threadIdx.x;
  const int d = x % DK;
  const float* U = Uws + bh * N * (long)DKDV + x;
  const float* A = Aws + bh * N * (long)DK + d;
  half_t* S = Sws + bh * N * (long)DKDV + x;
  float s = 0.f;
  int n = 0;
  for (; n + 8 <= N; n += 8) {
    float u[8], a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u[i] = U[(long)(n + i) * DKDV];
      a[i] = A[(long)(n + i) * DK];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      S[(long)(n + i) * DKDV] = (half_t)s;
      s = a[i] * s + u[i];
    }
  }
  for (; n < N; ++n) {
    S[(long)n * DKDV] = (half_t)s;
    s = A[(long)n * DK] * s + U[(long)n * DKDV];
  }
}

// ===========================================================================
// Phase 3: chunk outputs. One workgroup per (chunk n, head h, batch b).
//   O = A V + Q^ S_n,   A = causal decayed score tile (in LDS, half)
// ===========================================================================
template <int DK, int DV, int C, typename InT>
__global__ __launch_bounds__(kThreads) void output_kernel(
    const InT* __restrict__ qp, const InT* __restrict__ kp, const InT* __restrict__ vp,
    const InT* __restrict__ gp, const half_t* __restrict__ Sws, InT* __restrict__ op, int T,
    int H, int N, int gh, int gw, DirPack dirs) {
  using G = Geo<DK, DV, C>;
  constexpr int CP = G::CP, NB = G::NB;
  constexpr int DMAX = DK > DV ? DK : DV;
  constexpr int VA = (C * G::VSTR > C * G::TSTR) ? C * G::VSTR : C * G::TSTR;
  __shared__ __attribute__((aligned(16))) float sAl[C][DK];      // g2, then 2^(g2)
  __shared__ __attribute__((aligned(16))) float sQt[C * DMAX];   // Q~ (f32), then O staging
  __shared__ __attribute__((aligned(16))) half_t sQ[C][G::KSTR];
  __shared__ __attribute__((aligned(16))) half_t sK[C][G::KSTR];
  __shared__ __attribute__((aligned(16))) half_t sKt[C][G::KSTR];  // K~ row-major
  __shared__ __attribute__((aligned(16))) half_t sQh[C][G::KSTR];  // Q^ row-major
  __shared__ __attribute__((aligned(16))) half_t sVA[VA];          // V rows, then A tile
  __shared__ __attribute__((aligned(16))) half_t sVt[DV][G::TSTR];
  __shared__ float sBnd[NB + 1][DK];
  __shared__ float sM[G::NPAIR > 0 ? G::NPAIR : 1][DK];
  __shared__ float sTot[G::NSEG][DK];
  __shared__ int sRow[C];
  half_t (*sV)[G::VSTR] = reinterpret_cast<half_t (*)[G::VSTR]>(sVA);
  half_t (*sA)[G::TSTR] = reinterpret_cast<half_t (*)[G::TSTR]>(sVA);

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int tok0 = n * C;
  const int L = min(C, T - tok0);
  if (tid < C) sRow[tid] = tid < L ? scan_to_raster(tok0 + tid, T, gh, gw, dirs.get(b)) : -1;
  __syncthreads();

  // -- load q, k, gk rows (dk) and v rows (dv); padding rows are zero
  for (int u = tid; u < C * (DK / 8); u += kThreads) {
    const int r = u / (DK / 8), c8 = (u % (DK / 8)) * 8;
    float g8[8];
    half8 q8, k8;
    if (sRow[r] >= 0) {
      const long row = ((long)b * T + sRow[r]) * H + h;
      load8(gp + row * DK + c8, g8);
      q8 = load8h(qp + row * DK + c8);
      k8 = load8h(kp + row * DK + c8);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) { g8[c] = 0.f; q8[c] = k8[c] = (half_t)0.f; }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sAl[r][c8 + c] = g8[c] * kLog2e;
    *reinterpret_cast<half8*>(&sQ[r][c8]) = q8;
    *reinterpret_cast<half8*>(&sK[r][c8]) = k8;
  }
  for (int u = tid; u < C * (DV / 8); u += kThreads) {
    const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
    half8 v8;
    if (sRow[r] >= 0) {
      const long row = ((long)b * T + sRow[r]) * H + h;
      v8 = load8h(vp + row * DV + c8);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v8[c] = (half_t)0.f;
    }
    *reinterpret_cast<half8*>(&sV[r][c8]) = v8;
  }
  __syncthreads();

  // -- cumsum; g2 -> per-token decay 2^(g2) in place; sub-block boundaries
  const int d = tid % DK, seg = tid / DK;
  float p[G::SEGLEN];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < G::SEGLEN; ++i) {
    const int t = seg * G::SEGLEN + i;
    const float g2 = sAl[t][d];
    run += g2;
    p[i] = run;
    sAl[t][d] = exp2f(g2);
  }
  sTot[seg][d] = run;
  // V transposed into [e][token] (reads sV, written before the last barrier)
  for (int u = tid; u < DV * (C / 8); u += kThreads) {
    const int e = u % DV, j8 = (u / DV) * 8;
    half8 x;
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = sV[j8 + c][e];
    *reinterpret_cast<half8*>(&sVt[e][j8]) = x;
  }
  if constexpr (CP > C) {
    for (int u = tid; u < DV * (CP - C); u += kThreads)
      sVt[u / (CP - C)][C + u % (CP - C)] = (half_t)0.f;
  }
  __syncthreads();
  float off = 0.f;
#pragma unroll
  for (int s = 0; s < G::NSEG; ++s)
    if (s < seg) off += sTot[s][d];
  if (seg == 0) sBnd[0][d] = 0.f;
  if (((seg + 1) * G::SEGLEN) % 16 == 0) sBnd[(seg + 1) * G::SEGLEN / 16][d] = off + run;
  __syncthreads();

  // -- factors: Q~ (f32), Q^ (half), K~ (half), and the pair factors m_IJ
  {
    const int I = (seg * G::SEGLEN) / 16;  // the segment lies in one sub-block
    const float beta = sBnd[I][d], eI = sBnd[I + 1][d];
    const float ebeta = exp2f(beta);
#pragma unroll
    for (int i = 0; i < G::SEGLEN; ++i) {
      const int t = seg * G::SEGLEN + i;
      const float bt = off + p[i];
      const float qt = (float)sQ[t][d] * exp2f(bt - beta);
      sQt[t * DK + d] = qt;
      sQh[t][d] = (half_t)(qt * ebeta);
      sKt[t][d] = (half_t)((float)sK[t][d] * exp2f(eI - bt));
    }
    if (seg == 0) {
      for (int I2 = 1; I2 < NB; ++I2)
        for (int J = 0; J < I2; ++J)
          sM[I2 * (I2 - 1) / 2 + J][d] = exp2f(sBnd[I2][d] - sBnd[J + 1][d]);
    }
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = 8 * (lane >> 4);

  // -- strict upper triangle of the tile (causal mask), padding columns included
  for (int u = tid; u < C * CP; u += kThreads) {
    const int row = u / CP, col = u % CP;
    if (col > row) sA[row][col] = (half_t)0.f;
  }

  // -- diagonal sub-blocks, exact: A_ij = sum_d q_i k_j prod_{r=j+1..i} 2^(g2_r)
  //    A wave owns one row index i of every diagonal sub-block at a time
  //    (rows {w, 7-w, 8+w, 15-w}: equal work per wave); a lane owns four key
  //    dims of one sub-block; j runs from i down to 0 carrying the product.
  {
    constexpr int LPB = DK / 4;  // lanes per sub-block
    const int I = lane / LPB, dq = lane % LPB;
    const bool active = I < NB;
#pragma unroll 1
    for (int ri = 0; ri < 4; ++ri) {
      const int i = (ri & 1) ? ((ri & 2) ? 15 - wave : 7 - wave) : ((ri & 2) ? 8 + wave : wave);
      float u4[4] = {0.f, 0.f, 0.f, 0.f};
      if (active) {
#pragma unroll
        for (int c = 0; c < 4; ++c) u4[c] = (float)sQ[16 * I + i][4 * dq + c];
      }
#pragma unroll 1
      for (int j = i; j >= 0; --j) {
        float acc = 0.f;
        if (active) {
          const half4 k4 = *reinterpret_cast<const half4*>(&sK[16 * I + j][4 * dq]);
          const floatx4 al = *reinterpret_cast<const floatx4*>(&sAl[16 * I + j][4 * dq]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc += u4[c] * (float)k4[c];
            u4[c] *= al[c];
          }
        }
#pragma unroll
        for (int o = LPB / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
        if (active && dq == 0) sA[16 * I + i][16 * I + j] = (half_t)acc;
      }
    }
  }

  // -- off-diagonal sub-blocks I > J on the matrix cores
  for (int pr = wave; pr < G::NPAIR; pr += 4) {
    int I = 1;
    while ((I + 1) * I / 2 <= pr) ++I;
    const int J = pr - I * (I - 1) / 2;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const int d0 = 32 * ks + lk;
      half8 a;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        a[c] = (half_t)(sQt[(16 * I + lr) * DK + d0 + c] * sM[pr][d0 + c]);
      const half8 bb = *reinterpret_cast<const half8*>(&sKt[16 * J + lr][d0]);
      acc = mfma16x16x32(a, bb, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sA[16 * I + 4 * (lane >> 4) + r][16 * J + lr] = (half_t)acc[r];
  }
  __syncthreads();

  // -- O = A V + Q^ S_n on the matrix cores; stage O (f32) in LDS
  constexpr int NE = DV / 16;
  const long bhn = ((long)b * H + h) * N + n;
  const half_t* Sb = Sws + bhn * (long)(DV * DK);
  float* sO = sQt;  // Q~ is no longer read
  for (int blk = wave; blk < NB * NE; blk += 4) {
    const int I = blk / NE, E = blk % NE;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < CP / 32; ++ks) {
      if (32 * ks <= 16 * I + 15) {
        const half8 a = *reinterpret_cast<const half8*>(&sA[16 * I + lr][32 * ks + lk]);
        const half8 bb = *reinterpret_cast<const half8*>(&sVt[16 * E + lr][32 * ks + lk]);
        acc = mfma16x16x32(a, bb, acc);
      }
    }
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const half8 a = *reinterpret_cast<const half8*>(&sQh[16 * I + lr][32 * ks + lk]);
      const half8 bb = load8h(Sb + (16 * E + lr) * DK + 32 * ks + lk);
      acc = mfma16x16x32(a, bb, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(16 * I + 4 * (lane >> 4) + r) * DV + 16 * E + lr] = acc[r];
  }
  __syncthreads();

  // -- scatter rows back to their raster positions
  for (int u = tid; u < C * (DV / 8); u += kThreads) {
    const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
    if (sRow[r] < 0) continue;
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = sO[r * DV + c8 + c];
    store8(op + (((long)b * T + sRow[r]) * H + h) * DV + c8, x);
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
                     reinterpret_cast<float*>(ws + w.off_U) + bhn * DK * DV,
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
  hipLaunchKernelGGL((output_kernel<DK, DV, C, InT>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     reinterpret_cast<const half_t*>(ws + w.off_S) + bhn * DK * DV,
                     static_cast<InT*>(o) + tok * DV, p.T, p.H, p.N, p.gh, p.gw, dirs);
  return hipGetLastError();
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
  w.off_U = 0;
  w.off_a = up(units * p.dk * p.dv * sizeof(float));
  w.off_S = w.off_a + up(units * p.dk * sizeof(float));
  w.total = w.off_S + up(units * p.dk * p.dv * sizeof(half_t));
  return w;
}

hipError_t launch_summaries(const Problem& p, int b0, int nb, const DirPack& dirs,
                            const void* k, const void* v, const void* gk, char* ws,
                            hipStream_t s) {
  GLA_DISPATCH(summaries_t, p, b0, nb, dirs, k, v, gk, ws, s);
}

hipError_t launch_scan(const Problem& p, int b0, int nb, char* ws, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const long bhn = (long)b0 * p.H * p.N;
  const int dkdv = p.dk * p.dv;
  dim3 grid(dkdv / kThreads, nb * p.H);
  hipLaunchKernelGGL(scan_kernel, grid, dim3(kThreads), 0, s,
                     reinterpret_cast<const float*>(ws + w.off_U) + bhn * dkdv,
                     reinterpret_cast<const float*>(ws + w.off_a) + bhn * p.dk,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhn * dkdv, p.N, p.dk, dkdv);
  return hipGetLastError();
}

hipError_t launch_outputs(const Problem& p, int b0, int nb, const DirPack& dirs,
                          const void* q, const void* k, const void* v, const void* gk,
                          void* o, const char* ws, hipStream_t s) {
  GLA_DISPATCH(outputs_t, p, b0, nb, dirs, q, k, v, gk, o, ws, s);
}

hipError_t launch_scan_perm(int32_t* perm, int gh, int gw, int dir, hipStream_t s) {
  const int T = gh * gw;
  hipLaunchKernelGGL(scan_perm_kernel, dim3((T + 255) / 256), dim3(256), 0, s, perm, T, gh, gw,
                     dir);
  return hipGetLastError();
}

}  // namespace gla
