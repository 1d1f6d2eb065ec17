// The chunk kernel (outputs of the three-phase schedule, and the whole
// forward in the single-pass schedule) and its launch templates. Included by
// gla_kernels.hip (plain outputs) and gla_gated.hip (outputs with the fused
// RMS-normalised SiLU output gate), so that the two sets of instantiations
// compile as separate units.
#pragma once

#include "gla_launch.h"
#include "gla_tile.h"

namespace gla {
namespace tile {

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
//   2. takes the state it enters, in two levels over segments of G chunks:
//        S_n = X + W (.) P,  X = sum_{s0 <= m < n} (prod_{m<j<n} a_j) (.) U_m,
//        W = prod_{s0 <= j < n} a_j,  P = state entering the segment
//      where P composes the aggregates (prod a, sum of decayed U) that the
//      last chunk of each earlier segment publishes (and the initial state);
//      the in-segment part X, W comes first, so the segment's last chunk
//      publishes its aggregate before it computes its intra-chunk part A V
//      (the other chunks compute theirs while the aggregates arrive);
//   3. adds the readout Q^ S_n and stores the outputs.
// ===========================================================================
template <int DK, int DV, int C, typename InT, bool kFused, bool kGate>
__global__ __launch_bounds__(kThreads, 4) void chunk_kernel(
    const InT* __restrict__ qp, const InT* __restrict__ kp, const InT* __restrict__ vp,
    const InT* __restrict__ gp, InT* __restrict__ op, half_t* __restrict__ Uws,
    float* __restrict__ Aws, half_t* __restrict__ Sws, float* __restrict__ GAws,
    unsigned* __restrict__ ctrl, const float* __restrict__ s0, float* __restrict__ sfin,
    const InT* __restrict__ zp, const float* __restrict__ nw, float eps, int T, int H, int N,
    int G, int nseg, int gh, int gw, DirPack dirs) {
  constexpr int NB = C / 16, NKS = DK / 32, NEL = 8 * NKS, NE = DV / 16, ND = DK / 16;
  constexpr int NPAIR = NB * (NB - 1) / 2;
  constexpr int DKDV = DK * DV;
  constexpr int KSTR = DK + 8;   // halves, rows of K~ (read along key dims)
  constexpr int VSTR = DV + 16;  // halves, rows of V (read transposed)
  constexpr int HSTR = DK + 16;  // halves, rows of K^ (read transposed)
  constexpr int SSTR = DV + 16;  // halves, rows of S (read transposed)
  constexpr int USTR = DV + 8;   // halves, rows of the U staging tile
  constexpr int OSTR = DV + 8;   // rows of the output staging tile
  // the single pass's plain half output is staged column-major (rows = value
  // columns, 8-byte stores from the accumulators) and read back as token rows
  // through the transposing LDS read: fewer LDS operations on its critical
  // path. Each store then covers half a token row, which costs the
  // throughput-bound three-phase kernel more than it saves; it, the gated
  // and the fp32 outputs keep token rows.
  constexpr bool kColO = kFused && !kGate && sizeof(InT) == 2;
  constexpr int OTSTR = C + 16;  // halves, rows of the column-major output tile
  constexpr int NGR = (DKDV / 8 + kThreads - 1) / kThreads;  // state groups of 8 per thread
  constexpr int LB = 4;  // predecessors per batch of look-back loads
  constexpr float kHalfRange = 8.f, kF32Range = 120.f;  // log2 decay per sub-block
  // K~ is dead once the score blocks are built; the output tile reuses it
  constexpr int KO0 = C * KSTR * 2, KO1 = kColO ? DV * OTSTR * 2 : C * OSTR * (int)sizeof(InT);
  constexpr int KO_BYTES = KO0 > KO1 ? KO0 : KO1;
  // one region in turn holds K^, the U staging tile and S (only S unfused)
  constexpr int X0 = DK * SSTR * 2, X1 = kFused ? C * HSTR * 2 : 0, X2 = kFused ? DK * USTR * 2 : 0;
  constexpr int X_BYTES = X0 > X1 ? (X0 > X2 ? X0 : X2) : (X1 > X2 ? X1 : X2);
  __shared__ __attribute__((aligned(16))) char sKO[KO_BYTES];
  __shared__ __attribute__((aligned(16))) half_t sV[C][VSTR];
  __shared__ __attribute__((aligned(16))) char sX[X_BYTES];
  __shared__ __attribute__((aligned(16))) float sTot[NB][DK], sS7[NB][DK];
  __shared__ __attribute__((aligned(16))) float sEb[NB][DK], sR1[NB][DK], sR2[NB][DK];
  __shared__ __attribute__((aligned(16))) float sM[NPAIR > 0 ? NPAIR : 1][DK];
  __shared__ __attribute__((aligned(16))) float sF[kFused ? NB : 1][DK];  // K^ = K~ * sF
  __shared__ float sAn[kFused ? DK : 1];
  __shared__ int sRow[C];
  __shared__ int sTier;
  __shared__ unsigned sDone, sPub;
  half_t (*sKt)[KSTR] = reinterpret_cast<half_t (*)[KSTR]>(sKO);
  InT (*sO)[OSTR] = reinterpret_cast<InT (*)[OSTR]>(sKO);
  half_t (*sOT)[OTSTR] = reinterpret_cast<half_t (*)[OTSTR]>(sKO);
  // output block (sub-block I, value block E) of this lane: rows 16I + 4lq + r,
  // column 16E + lr
  auto stage_out = [&](const floatx4& acc, int E) {
    const int I = threadIdx.x >> 6, lq = (threadIdx.x >> 4) & 3, lr = threadIdx.x & 15;
    if constexpr (kColO) {
      half4 hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (half_t)acc[r];
      *reinterpret_cast<half4*>(&sOT[16 * E + lr][16 * I + 4 * lq]) = hv;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[16 * I + 4 * lq + r][16 * E + lr] = (InT)acc[r];
    }
  };
  half_t (*sS)[SSTR] = reinterpret_cast<half_t (*)[SSTR]>(sX);
  half_t (*sKh)[HSTR] = reinterpret_cast<half_t (*)[HSTR]>(sX);
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
  const int dir = dirs.get(b);
  // the row table (for the scatter) and the flags below are first read after
  // the barrier that follows the cumulative sums
  chunk_rows<C>(sRow, n * C, T, gh, gw, dir);
  if (tid == 0) sTier = 0, sPub = 0u;

  // -- this wave's token rows of q, k, gk in the operand layout (waves past
  // the last sub-block load a padding row too: no branch around the loads)
  const bool owner = wave < NB;
  const int I = wave, t = 16 * I + lr;
  float qf[NEL], kf[NEL], sc[NEL];
  bool pad;  // this lane's token row is padding
  {
    const int rr = owner ? token_row(n * C + t, T, gh, gw, dir) : -1;
    const long row = rr >= 0 ? ((long)b * T + rr) * H + h : -1;
    pad = row < 0;
    load_row<DK, NKS>(qp, row, lk, qf);
    load_row<DK, NKS>(kp, row, lk, kf);
    load_row<DK, NKS>(gp, row, lk, sc);
  }
  // -- the entering state (stored [dk][dv], staged as rows sS[d][e]; three-
  // phase schedule only) and the chunk's V rows, through LDS; every load is
  // issued before the first LDS write that waits on one
  constexpr int NSIT = kFused ? 1 : (DKDV / 8 + kThreads - 1) / kThreads;
  half8 h8[NSIT];
  if constexpr (!kFused) {
    const half_t* Sb = Sws + bhn * (long)DKDV;
#pragma unroll
    for (int it = 0; it < NSIT; ++it) h8[it] = load8h(Sb + 8 * ((tid + kThreads * it) % (DKDV / 8)));
  }
  load_v<DV, C, VSTR>(vp, n * C, T, gh, gw, dir, (long)b * T, H, h, sV);
  if constexpr (!kFused) {
#pragma unroll
    for (int it = 0; it < NSIT; ++it) {
      const int u = tid + kThreads * it;
      if (u < DKDV / 8) {
        const int d = u / (DV / 8), e8 = (u % (DV / 8)) * 8;
        *reinterpret_cast<half8*>(&sS[d][e8]) = h8[it];
      }
    }
  }

  if ((n + 1) * C > T) {  // the chain's last chunk: zero the padding rows
    zero_row<NEL>(pad, qf);
    zero_row<NEL>(pad, kf);
    zero_row<NEL>(pad, sc);
  }
  // -- in-sub-block inclusive cumsum along tokens (DPP row scan)
  if (owner) {
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(sc[e]) * kLog2e;
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
    float tots[NB];  // every sub-block's total, read together
#pragma unroll
    for (int J = 0; J < NB; ++J) tots[J] = sTot[J][d];
    const float s7 = sS7[I2][d];
    float beta = 0.f, tot = 0.f, after = 0.f;  // totals before, of and after I2
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < I2) beta += tots[J];
      else if (J == I2) tot = tots[J];
      else after += tots[J];
    }
    sEb[I2][d] = fexp2(beta);
    sR1[I2][d] = fexp2(-s7);
    sR2[I2][d] = fexp2(s7 - tot);
    float acc = 0.f;  // log2 of m_{I2,J} for J = I2-1, I2-2, ...
#pragma unroll
    for (int J = NB - 2; J >= 0; --J) {
      if (J < I2) {
        sM[I2 * (I2 - 1) / 2 + J][d] = fexp2(acc);
        acc += tots[J];
      }
    }
    const float range = -tot;
    if (!(range <= kF32Range)) atomicMax(&sTier, 2);
    else if (!(range <= kHalfRange)) atomicMax(&sTier, 1);
    if constexpr (kFused) {
      sF[I2][d] = fexp2(after);
      if (I2 == NB - 1) sAn[d] = fexp2(beta + tot);  // a_n = 2^(chunk total)
    }
  }
  __syncthreads();
  // -- per-element factors; K~ goes to LDS for the other sub-blocks, and in
  // one pass K^ = K~ 2^(totals of the later sub-blocks), for U
  float qt[NEL], kt[NEL];
  if (owner) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float tt[8], ff[8];
      lds8(&sTot[I][32 * ks + lk], tt);
      if constexpr (kFused) lds8(&sF[I][32 * ks + lk], ff);
      half8 k8, kh8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = 8 * ks + c;
        qt[e] = qf[e] * fexp2(sc[e]);
        kt[e] = kf[e] * fexp2(tt[c] - sc[e]);
        k8[c] = (half_t)kt[e];
        if constexpr (kFused) kh8[c] = (half_t)(kt[e] * ff[c]);
      }
      *reinterpret_cast<half8*>(&sKt[t][32 * ks + lk]) = k8;
      if constexpr (kFused) *reinterpret_cast<half8*>(&sKh[t][32 * ks + lk]) = kh8;
    }
  }
  __syncthreads();

  unsigned* cw = nullptr;  // this chain's control words
  // this chain's summaries and segment aggregates (single pass only)
  const __amdgpu_buffer_rsrc_t rU = coh_rsrc(Uws + bh * N * DKDV, (long)N * DKDV);
  const __amdgpu_buffer_rsrc_t rS = coh_rsrc(Sws + bh * nseg * DKDV, (long)nseg * DKDV);
  if constexpr (kFused) {
    cw = ctrl + kCtrlHeader + bh * (long)(N + nseg + 1);
    // -- U_n^T = V^T K^ in 16x16 blocks, staged as rows of key dims (the
    // tile stays in LDS until the segment's aggregate is built), published
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
          const half4 a = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
          const half4 bb = ld_tr<HSTR, 4>(&sKh[16 * J][16 * D]);
          uacc[i] = mfma16x16x16(a, bb, uacc[i]);
        }
      }
    }
    __syncthreads();  // K^ is no longer read: the region becomes the U staging tile
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
        st_coh(rU, n * DKDV + x8, *reinterpret_cast<const half8*>(&sU[x8 / DV][x8 % DV]));
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
            const half4 sb = ld_tr<SSTR, 8>(&sS[32 * ks + 4 * hh][16 * E]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            acc = mfma16x16x16(qa, sb, acc);
          }
        }
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            acc = mfma16x16x16(A[J], vb, acc);
          }
        }
        stage_out(acc, E);
      }
    }
  } else {
    // -- the entering state, in-segment part: X and W
    const int seg = n / G, n0 = seg * G, nlast = min(n0 + G, N) - 1;
    const bool agg = n == nlast && seg < nseg - 1;  // publishes the segment's aggregate
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
          const int mj = m - j >= n0 ? m - j : n0;
          u[g][j] = ld_coh(rU, mj * DKDV + x8);
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
          consume(u[g][j], a[g][j]);
        }
      }
    }
    // -- the last chunk of a segment publishes the segment's aggregate
    if (agg) {
      const long gs = bh * nseg + seg;
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
        if (x8 < DKDV) {
          half8 ag;
          const half8 un = *reinterpret_cast<const half8*>(&sU[d][x8 % DV]);  // own U_n
#pragma unroll
          for (int c = 0; c < 8; ++c) ag[c] = (half_t)(sAn[d] * xs[g][c] + (float)un[c]);
          st_coh(rS, seg * DKDV + x8, ag);
        }
      }
      // the segment's decay: the weight the look-back accumulated, times a_n
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
        if (x8 < DKDV && x8 % DV == 0) st_dev(GAws + gs * DK + d, wv[g] * sAn[d]);
      }
    }
    // -- intra-chunk part, while the aggregate's stores complete and the
    // earlier segments publish: O_I = sum_{J<=I} A_IJ V_J
    floatx4 oacc[NE];
#pragma unroll
    for (int E = 0; E < NE; ++E) {
      oacc[E] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (owner) {
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            oacc[E] = mfma16x16x16(A[J], vb, oacc[E]);
          }
        }
      }
    }
    if (agg) publish_wave(cw + N + seg, &sPub);
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
          const int sj = s2 - j >= 0 ? s2 - j : 0;
          u[g][j] = ld_coh(rS, sj * DKDV + x8);
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
          consume(u[g][j], a[g][j]);
        }
      }
    }
    // the chain's last chunk also returns the state after it, a_n S_n + U_n:
    // its own U_n comes from the staging tile, read before S overwrites it
    const bool fin = sfin != nullptr && n == N - 1;
    half8 ul[NGR];
    if (fin) {
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
        ul[g] = *reinterpret_cast<const half8*>(&sU[x8 / DV][x8 % DV]);
      }
      __syncthreads();
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
        if (fin) {
          float f[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) f[c] = sAn[d] * xs[g][c] + (float)ul[g][c];
          store_f8(sfin + bh * DKDV + x8, f);
        }
        half8 s8;
#pragma unroll
        for (int c = 0; c < 8; ++c) s8[c] = (half_t)xs[g][c];
        *reinterpret_cast<half8*>(&sS[d][x8 % DV]) = s8;
      }
    }
    __syncthreads();  // S_n complete in LDS; every read of published data done
    // -- readout, on the same accumulation chains: O_I += Q^_I S_n
    if (owner) {
#pragma unroll
      for (int E = 0; E < NE; ++E) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb = ld_tr<SSTR, 8>(&sS[32 * ks + 4 * hh][16 * E]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            oacc[E] = mfma16x16x16(qa, sb, oacc[E]);
          }
        }
        stage_out(oacc[E], E);
      }
    }
  }
  __syncthreads();

  // -- scatter rows back to their raster positions; with the output gate,
  // each row of dv values becomes o / sqrt(mean(o^2) + eps) * w * silu(z)
  // (its dv/8 lanes are neighbours and reduce the sum of squares by shuffles)
  constexpr int LPR = DV / 8;  // lanes per output row
  if constexpr (kColO) {
    // unit (token block tb, value half eh): lane (lr, lq) takes token
    // 16tb + lr, values 32eh + 8lq + 0..7, in two transposing reads
    constexpr int NTB = C / 16, NU = NTB * (DV / 32);
    for (int u = wave; u < NU; u += kThreads / 64) {
      const int tb = u % NTB, eh = u / NTB, t = 16 * tb + lr;
      const half4 lo = ld_tr<OTSTR, 8>(&sOT[32 * eh][16 * tb]);
      const half4 hi = ld_tr<OTSTR, 8>(&sOT[32 * eh + 4][16 * tb]);
      if (sRow[t] >= 0)
        *reinterpret_cast<half8*>(op + (((long)b * T + sRow[t]) * H + h) * DV + 32 * eh + 8 * lq) =
            __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  for (int u = tid; u < (kColO ? 0 : C * LPR); u += kThreads) {
    const int r = u / LPR, c8 = (u % LPR) * 8;
    const long orow = ((long)b * T + (sRow[r] >= 0 ? sRow[r] : 0)) * H + h;
    if constexpr (!kGate) {
      if (sRow[r] >= 0) copy8(op + orow * DV + c8, &sO[r][c8]);
      continue;
    }
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = (float)sO[r][c8 + c];
    if constexpr (kGate) {
      float z[8], wn[8];
      load8(zp + orow * DV + c8, z);
      load_f8(nw + c8, wn);
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss += x[c] * x[c];
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float sg = __builtin_amdgcn_rcpf(1.f + fexp2(-z[c] * kLog2e));  // sigmoid(z)
        x[c] *= inv * wn[c] * z[c] * sg;
      }
    }
    if (sRow[r] >= 0) store8(op + orow * DV + c8, x);
  }
  if constexpr (kFused) {
    // -- this chunk is done reading what its chain published: count it; the
    // last chunk of the chain to finish clears the chain's control words (off
    // the critical path, after the outputs are on their way)
    if (tid == 0) sDone = atomicAdd(ctrl + kCtrlHeader + bh * (long)(N + nseg + 1) + N + nseg, 1u);
    __syncthreads();
    if (sDone == (unsigned)(N - 1)) {
      unsigned* cw = ctrl + kCtrlHeader + bh * (long)(N + nseg + 1);
      for (int i = tid; i < N + nseg + 1; i += kThreads) cw[i] = 0u;
    }
  }
}

template <int DK, int DV, int C, typename InT, bool kGate>
hipError_t outputs_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                     const void* k, const void* v, const void* gk, void* o, const char* ws,
                     const Epilogue& epi, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  dim3 grid(p.N, p.H, nb);
  hipLaunchKernelGGL((chunk_kernel<DK, DV, C, InT, false, kGate>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     static_cast<InT*>(o) + tok * DV, nullptr, nullptr,
                     const_cast<half_t*>(reinterpret_cast<const half_t*>(ws + w.off_S)) +
                         bhn * DK * DV,
                     nullptr, nullptr, nullptr, nullptr,
                     kGate ? static_cast<const InT*>(epi.gate) + tok * DV : nullptr,
                     epi.weight, epi.eps, p.T, p.H, p.N, 1, 1, p.gh, p.gw, dirs);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename InT, bool kGate>
hipError_t onepass_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                     const void* k, const void* v, const void* gk, void* o, char* ws,
                     const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const Segments sg = onepass_segments(p.N);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  const long bhs = (long)b0 * p.H * sg.nseg;
  const long st = (long)b0 * p.H * DK * DV;
  // chain-major: every chunk of one (batch, head) before the next chain
  dim3 grid((unsigned)((long)nb * p.H * p.N));
  hipLaunchKernelGGL((chunk_kernel<DK, DV, C, InT, true, kGate>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     static_cast<InT*>(o) + tok * DV,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhn * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_a) + bhn * DK,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhs * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_g) + bhs * DK,
                     reinterpret_cast<unsigned*>(ws), s0 ? s0 + st : nullptr,
                     sfin ? sfin + st : nullptr,
                     kGate ? static_cast<const InT*>(epi.gate) + tok * DV : nullptr, epi.weight,
                     epi.eps, p.T, p.H, p.N, sg.G, sg.nseg, p.gh, p.gw, dirs);
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

}  // namespace tile
}  // namespace gla
