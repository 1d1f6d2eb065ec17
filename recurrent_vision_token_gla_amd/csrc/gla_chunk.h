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
// Chunk outputs. One workgroup per (chunk n, head h, batch b), or VS of
// them, each on DV of the head's VS DV value columns (VS > 1: the single
// pass's value split; every column of the state is its own recurrence, so
// the workgroups share nothing but their q, k, gk inputs).
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
// Each wave picks the diagonal block's arithmetic from its own 16 tokens:
// half operands while no key dim decays by more than 2^8 over the block and
// max(|Q~|, |K~|) * 2^range stays within 2^15, float operands while the range
// is within 2^120 and those factors stay finite, and beyond that a direct
// float sum of every entry from 2^(s_i - s_j) (q and k read again). Score
// entries beyond 2^14 in magnitude make the wave divide its score blocks by a
// power of two sigA, undone on the accumulators (the product with V is
// linear).
//
// The three-phase entering state S_n arrives as half rows divided by their
// power-of-two scales sigS[d] >= 1. The readout folds sigS[d] / max_d sigS
// into Q^ (a factor <= 1) and multiplies the accumulators by max_d sigS.
//
// kFused = false: phase 3 of three; S_n comes from the boundary scan.
// kFused = true: the whole forward in one pass (the chunk summary, the
// boundary state and the outputs). Workgroups are numbered chunk-major (chunk
// n of every chain, then chunk n + 1), so a chunk only ever waits on chunks
// of lower index, which were dispatched earlier, and the workgroups resident
// at any time are the earliest unfinished chunks of every chain rather than
// whole chains waiting on one another's publications. Each chunk
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
template <int DK, int DV, int C, typename InT, bool kFused, bool kGate, int GR = 1, int VS = 1>
__global__ __launch_bounds__(kThreads * GR, 4 / GR) void chunk_kernel(
    const InT* __restrict__ qp, const InT* __restrict__ kp, const InT* __restrict__ vp,
    const InT* __restrict__ gp, InT* __restrict__ op, half_t* __restrict__ Uws,
    float* __restrict__ Aws, half_t* __restrict__ Sws, const float* __restrict__ SigS,
    float* __restrict__ GAws, unsigned* __restrict__ ctrl, const float* s0, float* sfin,
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
  constexpr int NGR = (DKDV / 8 + kThreads - 1) / kThreads;  // state groups of 8 per thread
  constexpr int LB = 4;  // predecessors per batch of look-back loads
  constexpr float kHalfRange = 8.f, kF32Range = 120.f;  // log2 decay per sub-block
  // K~ is dead once the score blocks are built; the output tile reuses it
  constexpr int KO0 = C * KSTR * 2, KO1 = C * OSTR * (int)sizeof(InT);
  constexpr int KO_BYTES = KO0 > KO1 ? KO0 : KO1;
  // one region in turn holds K^, the U staging tile and S (only S unfused)
  constexpr int X0 = DK * SSTR * 2, X1 = kFused ? C * HSTR * 2 : 0, X2 = kFused ? DK * USTR * 2 : 0;
  constexpr int X_BYTES = X0 > X1 ? (X0 > X2 ? X0 : X2) : (X1 > X2 ? X1 : X2);
  // LDS: one block of the tiles below per chunk of the workgroup (GR of them)
  constexpr int TAB = NB * DK * 4;  // bytes of one [sub-block][key dim] float table
  constexpr int L_V = lds_round(KO_BYTES), L_X = lds_round(L_V + C * VSTR * 2);
  constexpr int L_TAB = lds_round(L_X + X_BYTES);  // sTot, sS7, sEb, sR1, sR2
  constexpr int L_M = L_TAB + 5 * TAB, L_F = L_M + (NPAIR > 0 ? NPAIR : 1) * DK * 4;
  constexpr int L_AN = L_F + (kFused ? NB : 1) * DK * 4, L_ROW = L_AN + (kFused ? DK : 1) * 4;
  constexpr int L_SIG = L_ROW + C * 4, L_RMAX = L_SIG + DK * 4;
  constexpr int L_SIGU = L_RMAX + (kFused ? DK : 1) * 4, L_W = L_SIGU + (kFused ? DK : 1) * 4;
  constexpr int PER = lds_round(L_W + 20);
  static_assert(GR * PER <= 160 * 1024, "the chunks of a workgroup exceed the LDS of a CU");
  __shared__ __attribute__((aligned(16))) char sL[GR * PER];
  __shared__ int sLook[2];  // runs: the look-back's result, for the whole workgroup
  const int grp = GR > 1 ? (int)threadIdx.x / kThreads : 0;  // this thread's chunk in the workgroup
  char* const lb = sL + grp * PER;
  char(&sKO)[KO_BYTES] = *reinterpret_cast<char(*)[KO_BYTES]>(lb);
  half_t(&sV)[C][VSTR] = *reinterpret_cast<half_t(*)[C][VSTR]>(lb + L_V);
  char(&sX)[X_BYTES] = *reinterpret_cast<char(*)[X_BYTES]>(lb + L_X);
  float(&sTot)[NB][DK] = *reinterpret_cast<float(*)[NB][DK]>(lb + L_TAB);
  float(&sS7)[NB][DK] = *reinterpret_cast<float(*)[NB][DK]>(lb + L_TAB + TAB);
  float(&sEb)[NB][DK] = *reinterpret_cast<float(*)[NB][DK]>(lb + L_TAB + 2 * TAB);
  float(&sR1)[NB][DK] = *reinterpret_cast<float(*)[NB][DK]>(lb + L_TAB + 3 * TAB);
  float(&sR2)[NB][DK] = *reinterpret_cast<float(*)[NB][DK]>(lb + L_TAB + 4 * TAB);
  float(&sM)[NPAIR > 0 ? NPAIR : 1][DK] =
      *reinterpret_cast<float(*)[NPAIR > 0 ? NPAIR : 1][DK]>(lb + L_M);
  float(&sF)[kFused ? NB : 1][DK] = *reinterpret_cast<float(*)[kFused ? NB : 1][DK]>(lb + L_F);  // K^ = K~ * sF
  float(&sAn)[kFused ? DK : 1] = *reinterpret_cast<float(*)[kFused ? DK : 1]>(lb + L_AN);
  int(&sRow)[C] = *reinterpret_cast<int(*)[C]>(lb + L_ROW);
  float(&sSig)[DK] = *reinterpret_cast<float(*)[DK]>(lb + L_SIG);  // row scales of S_n
  // single pass: row maxima and row scales of U_n
  unsigned(&sRowMax)[kFused ? DK : 1] = *reinterpret_cast<unsigned(*)[kFused ? DK : 1]>(lb + L_RMAX);
  float(&sSigU)[kFused ? DK : 1] = *reinterpret_cast<float(*)[kFused ? DK : 1]>(lb + L_SIGU);
  float& sSigMax = *reinterpret_cast<float*>(lb + L_W);
  unsigned& sDone = *reinterpret_cast<unsigned*>(lb + L_W + 4);
  unsigned& sPub = *reinterpret_cast<unsigned*>(lb + L_W + 8);
  unsigned& sPub2 = *reinterpret_cast<unsigned*>(lb + L_W + 12);
  // single pass and runs: the largest row scale of S_n as float bits (it
  // shares sSigMax's word), and whether any entry of U_n reached the half
  // range; both are rare, so their common case costs one wave vote each
  unsigned& sSigMaxBits = *reinterpret_cast<unsigned*>(lb + L_W);
  unsigned& sBigU = *reinterpret_cast<unsigned*>(lb + L_W + 16);
  half_t (*sKt)[KSTR] = reinterpret_cast<half_t (*)[KSTR]>(sKO);
  InT (*sO)[OSTR] = reinterpret_cast<InT (*)[OSTR]>(sKO);
  // The outputs are produced transposed (O^T = V^T A^T + S^T Q^T: the same
  // operand registers with the two operands swapped), so that each lane holds
  // four consecutive value columns 16E + 4lq + r of its token 16I + lr and
  // stages them with one 8-byte (16-byte for float) LDS write into token rows.
  auto stage_out = [&](const floatx4& acc, int E) {
    const int I = (threadIdx.x >> 6) % 4, lq = (threadIdx.x >> 4) & 3, lr = threadIdx.x & 15;
    if constexpr (sizeof(InT) == 2) {
      *reinterpret_cast<half4*>(&sO[16 * I + lr][16 * E + 4 * lq]) = cvt4(acc);
    } else {
      *reinterpret_cast<floatx4*>(&sO[16 * I + lr][16 * E + 4 * lq]) = acc;
    }
  };
  half_t (*sS)[SSTR] = reinterpret_cast<half_t (*)[SSTR]>(sX);
  half_t (*sKh)[HSTR] = reinterpret_cast<half_t (*)[HSTR]>(sX);
  half_t (*sU)[USTR] = reinterpret_cast<half_t (*)[USTR]>(sX);
  // runs: the state after the first `upto` chunks of the workgroup's run
  // when it enters at zero, x = sum_{m < upto} (prod_{m < i < upto} a_i) U_m
  // (elements x8..x8+7 of row d = x8 / DV, from the chunks' U tiles in LDS),
  // and the decay w = prod_{m < upto} a_m of that row
  auto run_prefix = [&](int upto, int x8, float (&x)[8], float& w) {
    const int d = x8 / DV;
    w = 1.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = 0.f;
#pragma unroll
    for (int m = 0; m < GR; ++m) {
      if (m < upto) {
        const char* lm = sL + m * PER;
        const float am = reinterpret_cast<const float*>(lm + L_AN)[d];
        const float su = reinterpret_cast<const float*>(lm + L_SIGU)[d];
        const half8 u = *reinterpret_cast<const half8*>(
            reinterpret_cast<const half_t*>(lm + L_X) + d * USTR + x8 % DV);
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = fmaf(su, (float)u[c], am * x[c]);
        w *= am;
      }
    }
  };

  int n, h, b;
  int run = 0;  // runs: this workgroup's run of GR chunks (nseg = runs per chain)
  if constexpr (GR > 1) {
    // run-major: every chain's run 0, then every chain's run 1, ...
    const int nch = (int)(gridDim.x / nseg);
    run = blockIdx.x / nch;
    const int ch = blockIdx.x - run * nch;
    n = run * GR + grp, h = ch % H, b = ch / H;
  } else if constexpr (kFused) {
    // chunk-major: chunk n of every chain, then chunk n + 1; with the value
    // columns split (VS > 1), each head is VS chains of DV columns
    const int nbh = (int)(gridDim.x / N);
    n = blockIdx.x / nbh;
    const int bh = blockIdx.x - n * nbh;
    h = bh % (H * VS), b = bh / (H * VS);
  } else {
    n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  }
  // this workgroup's chain (b, h) of B x (H VS) chains, its head hr and its
  // value columns vs DV .. vs DV + DV - 1 of that head's VS DV
  const long bh = (long)b * H * VS + h, bhn = bh * N + n;
  const int hr = h / VS, vs = h - hr * VS;
  constexpr int VP = DV * VS;
  // element (d, e) of this chain's state in a [B][H][DK][VS DV] state array
  auto st_at = [&](int d, int e) { return (((long)b * H + hr) * DK + d) * VP + vs * DV + e; };
  const int tid = GR > 1 ? (int)threadIdx.x % kThreads : (int)threadIdx.x;  // within the chunk
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = 8 * lq;
  const int dir = dirs.get(b);
  // the row table (for the scatter) and the flags below are first read after
  // the barrier that follows the cumulative sums
  chunk_rows<C>(sRow, n * C, T, gh, gw, dir, tid);
  if (tid == 0) sPub = 0u, sPub2 = 0u;
  if (kFused && tid == 0) sSigMaxBits = 0x3f800000u, sBigU = 0u;  // 1.0f; none
  if (kFused && tid < DK) sRowMax[tid] = 0u;

  // -- this wave's token rows of q, k, gk in the operand layout (waves past
  // the last sub-block load a padding row too: no branch around the loads)
  const bool owner = wave < NB;
  const int I = wave, t = 16 * I + lr;
  RawRow<InT, NKS> qr, kr, gr;  // as loaded, converted where consumed
  float sc[NEL];
  bool pad;  // this lane's token row is padding
  {
    const int rr = owner ? token_row(n * C + t, T, gh, gw, dir) : -1;
    const long row = rr >= 0 ? ((long)b * T + rr) * H + hr : -1;
    pad = row < 0;
    qr.load(qp, row, DK, lk);
    kr.load(kp, row, DK, lk);
    gr.load(gp, row, DK, lk);
  }
  // -- the row scales and the entering state (stored [dk][dv], staged as
  // rows sS[d][e]; three-phase schedule only) and the chunk's V rows, all
  // loaded now; the state and (see kDeferV) the V rows are written to LDS
  // after the decay scan, which so waits only for the q, k, gk rows issued
  // before them
  constexpr int NSIT = kFused ? 1 : (DKDV / 8 + kThreads - 1) / kThreads;
  half8 h8[NSIT];
  float sig_d = 1.f;  // thread d < DK: row scale of S_n row d
  if constexpr (!kFused) {
    sig_d = SigS[bhn * DK + (tid % DK)];
    const half_t* Sb = Sws + bhn * (long)DKDV;
#pragma unroll
    for (int it = 0; it < NSIT; ++it) h8[it] = load8h(Sb + 8 * ((tid + kThreads * it) % (DKDV / 8)));
  }
  VRows<DV, C, VSTR, InT> vrows;
  vrows.load(vp + vs * DV, n * C, T, gh, gw, dir, (long)b * T, H, hr, VP, tid);
  // (three-phase kernels with half inputs; with float inputs and in the
  // runs kernel there are no registers to spare, and the single pass gains
  // nothing measurable from it: their V rows go to LDS at once)
  constexpr bool kDeferV = sizeof(InT) == 2 && GR == 1 && !kFused;
  if constexpr (!kDeferV) vrows.store(n * C, T, sV, tid);

  if ((n + 1) * C > T) {  // the chain's last chunk: zero the padding rows
    qr.zero_if(pad);
    kr.zero_if(pad);
    gr.zero_if(pad);
  }
  // -- in-sub-block inclusive cumsum along tokens (DPP row scan), in log2
  if (owner) {
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(mulw(gr[e], kLog2e));
    if ((lr | 8) == 15) {  // lr 15 or 7: one compare, no branch between the scan's steps
#pragma unroll
      for (int e = 0; e < NEL; ++e) {
        const int d = 32 * (e / 8) + lk + (e % 8);
        if (lr == 15) sTot[I][d] = sc[e];
        else sS7[I][d] = sc[e];
      }
    }
  }
  if constexpr (!kFused) {
#pragma unroll
    for (int it = 0; it < NSIT; ++it) {
      const int u = tid + kThreads * it;
      if (u < DKDV / 8) {
        const int d = u / (DV / 8), e8 = (u % (DV / 8)) * 8;
        *reinterpret_cast<half8*>(&sS[d][e8]) = h8[it];
      }
    }
    if (tid < DK) sSig[tid] = sig_d;
  }
  if constexpr (kDeferV) vrows.store(n * C, T, sV, tid);
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
    if constexpr (kFused) {
      sEb[I2][d] = fexp2(beta);
    } else {
      // Q^ factor 2^beta * sigS[d] / max sigS (the accumulators take max sigS)
      const float sg = sSig[d];
      const float smax = __any(sg != 1.f) ? group_max<DK>(sg) : 1.f;
      if (tid == 0) sSigMax = smax;
      sEb[I2][d] = fexp2(beta) * sg * inv_scale(smax);
    }
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
    if constexpr (kFused) {
      sF[I2][d] = fexp2(after);
      if (I2 == NB - 1) sAn[d] = fexp2(beta + tot);  // a_n = 2^(chunk total)
    }
  }
  __syncthreads();
  // -- per-element factors; K~ goes to LDS for the other sub-blocks, and in
  // one pass K^ = K~ 2^(totals of the later sub-blocks), for U
  float qt[NEL], kt[NEL];
  // this lane's decay range over its sub-block (log2) and max(|Q~|, |K~|);
  // the totals are <= 0, so the largest magnitude is the largest bit pattern
  float rng = 0.f, bigt = 0.f;
  if (owner) {
    unsigned rbits = 0u;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float tt[8], ff[8];
      lds8(&sTot[I][32 * ks + lk], tt);
#pragma unroll
      for (int c = 0; c < 8; c += 2)
        rbits = max(rbits, max(__float_as_uint(tt[c]), __float_as_uint(tt[c + 1])));
      if constexpr (kFused) lds8(&sF[I][32 * ks + lk], ff);
      half8 k8, kh8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = 8 * ks + c;
        qt[e] = mulw(qr[e], fexp2(sc[e]));
        kt[e] = mulw(kr[e], fexp2(tt[c] - sc[e]));
        bigt = max3f(bigt, fabsf(qt[e]), fabsf(kt[e]));
        k8[c] = (half_t)kt[e];
        if constexpr (kFused) kh8[c] = (half_t)(kt[e] * ff[c]);
      }
      *reinterpret_cast<half8*>(&sKt[t][32 * ks + lk]) = k8;
      if constexpr (kFused) *reinterpret_cast<half8*>(&sKh[t][32 * ks + lk]) = kh8;
    }
    rng = __uint_as_float(rbits & 0x7fffffffu);
  }
  __syncthreads();

  unsigned* cw = nullptr;  // this chain's control words
  // this chain's summaries and segment aggregates (single pass), or its runs'
  // aggregates and inclusive states (runs; nseg runs per chain)
  const long nU = GR > 1 ? nseg : N;
  const __amdgpu_buffer_rsrc_t rU = coh_rsrc(Uws + bh * nU * DKDV, nU * DKDV);
  const __amdgpu_buffer_rsrc_t rS = coh_rsrc(Sws + bh * nseg * DKDV, (long)nseg * DKDV);
  if constexpr (kFused) {
    cw = ctrl + kCtrlHeader + bh * (long)(GR > 1 ? nseg + 1 : N + nseg + 1);
    // -- U_n^T = V^T K^ in 16x16 blocks, staged as rows of key dims (the
    // tile stays in LDS until the segment's aggregate is built), published
    constexpr int NBLK = NE * ND, BPW = (NBLK + 3) / 4;
    floatx4 uacc[BPW];
    float um[BPW];  // this lane's largest |entry| of each block
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      uacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      um[i] = 0.f;
      if (blk < NBLK) {
        const int E = blk / ND, D = blk % ND;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          const half4 a = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
          const half4 bb = ld_tr<HSTR, 4>(&sKh[16 * J][16 * D]);
          uacc[i] = mfma16x16x16(a, bb, uacc[i]);
        }
        um[i] = fmaxf(fmaxf(fabsf(uacc[i][0]), fabsf(uacc[i][1])),
                      fmaxf(fabsf(uacc[i][2]), fabsf(uacc[i][3])));
      }
    }
    // row maxima only from waves with an entry of 2^14 or more: a row whose
    // maximum is below that has scale 1 whatever is posted, and a row whose
    // maximum is not gets that maximum from the wave holding it
    float uw = 0.f;
#pragma unroll
    for (int i = 0; i < BPW; ++i) uw = fmaxf(uw, um[i]);
    if (__any(uw >= kRowRange)) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int blk = wave + 4 * i;
        if (blk < NBLK) atomicMax(&sRowMax[16 * (blk % ND) + lr], __float_as_uint(um[i]));
      }
      if (lane == 0) sBigU = 1u;
    }
    __syncthreads();  // K^ is no longer read: the region becomes the U staging tile
    const bool scale_u = sBigU != 0u;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      if (blk < NBLK) {
        const int E = blk / ND, D = blk % ND;
        floatx4 x = uacc[i];
        if (scale_u) x *= inv_scale(row_scale(__uint_as_float(sRowMax[16 * D + lr])));
        *reinterpret_cast<half4*>(&sU[16 * D + lr][16 * E + 4 * lq]) = cvt4(x);
      }
    }
    __syncthreads();
    if constexpr (GR == 1) {
      // wave 0 alone stores and flags U_n (rows divided by their scales), the
      // row scales and a_n, so that the other waves go on to their score
      // blocks without waiting for the stores to complete
      if (wave == 0) {
        for (int x8 = 8 * lane; x8 < DKDV; x8 += 8 * 64)
          st_coh(rU, n * DKDV + x8, *reinterpret_cast<const half8*>(&sU[x8 / DV][x8 % DV]));
        for (int d = lane; d < DK; d += 64) {
          const float sg = scale_u ? row_scale(__uint_as_float(sRowMax[d])) : 1.f;
          sSigU[d] = sg;
          st_dev2(Aws + 2 * (bhn * DK + d), sAn[d], sg);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_store(cw + n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      if (tid < DK) sSigU[tid] = scale_u ? row_scale(__uint_as_float(sRowMax[tid])) : 1.f;
      __syncthreads();  // every chunk's U_n, a_n and row scales are in LDS
      // the run's last chunk publishes the run's aggregate (the state after
      // the run when it enters at zero, and the run's decay); chunks past the
      // chain's end are padding (a = 1, U = 0), so every run has GR chunks
      if (grp == GR - 1 && run > 0) {
#pragma unroll
        for (int g = 0; g < NGR; ++g) {
          const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
          if (x8 < DKDV) {
            float x[8], w, m = 0.f;
            run_prefix(GR, x8, x, w);
#pragma unroll
            for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(x[c]));
            // the DV/8 neighbouring lanes of row d agree on its scale
            const float sg = row_scale(DV == 64 ? group_max<8>(m) : group_max<4>(m));
            const float inv = inv_scale(sg);
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] *= inv;
            st_coh(rU, run * DKDV + x8, cvt8(x));
            if (x8 % DV == 0) st_dev2(Aws + 2 * ((bh * nseg + run) * DK + d), w, sg);
          }
        }
        publish_wave(cw + run, &sPub, kStAgg);
      }
    }
  }

  half4 A[NB];
  half8 qh[NKS];
  float sigA = 1.f;  // this wave's score blocks are stored divided by sigA
  if (owner) {
    // the diagonal operands are Q~ 2^(-s_7) = q 2^(s_i - s_7) and
    // K~ 2^(s_7 - tot) = k 2^(s_7 - s_j), each at most max(|Q~|, |K~|)
    // 2^range in magnitude
    const float amp = bigt * fexp2(fminf(rng, 127.f));
    const int tier = __all(rng <= kHalfRange && amp <= 32768.f)  ? 0
                     : __all(rng <= kF32Range && amp < 0x1p126f) ? 1
                                                                  : 2;
    // -- diagonal sub-block, transposed: acc[r] = A[i = lr][j = 4*lq + r]
    floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
    if (tier == 0) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float r1[8], r2[8], qa[8], ka[8];
        lds8(&sR1[I][32 * ks + lk], r1);
        lds8(&sR2[I][32 * ks + lk], r2);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          qa[c] = qt[8 * ks + c] * r1[c];
          ka[c] = kt[8 * ks + c] * r2[c];
        }
        dacc = mfma16x16x32(cvt8(ka), cvt8(qa), dacc);
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
      // every entry directly: A_ij = sum_d q_i k_j 2^(s_i - s_j), with this
      // lane's q and k rows read again, eight dims at a time (keeping them
      // in registers through the common tiers would cost more than this
      // rare reload)
      const int rr = token_row(n * C + t, T, gh, gw, dir);
      const long row = rr >= 0 ? ((long)b * T + rr) * H + hr : -1;
      float part[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) part[j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        RawRow<InT, 1> q2, k2;
        q2.load(qp + 32 * ks, row, DK, lk);
        k2.load(kp + 32 * ks, row, DK, lk);
        q2.zero_if(row < 0);
        k2.zero_if(row < 0);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float qv = q2[c], kv = k2[c], sv = sc[8 * ks + c];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float kj = __shfl(kv, (lane & 48) | j);
            const float sj = __shfl(sv, (lane & 48) | j);
            part[j] += qv * kj * fexp2(sv - sj);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float pj = part[j];
        pj += __shfl_xor(pj, 16);
        pj += __shfl_xor(pj, 32);
        if ((j >> 2) == lq) dacc[j & 3] = pj;
      }
    }
    floatx4 Af[NB];  // score blocks in float, before the cast to half
#pragma unroll
    for (int r = 0; r < 4; ++r) dacc[r] = (4 * lq + r <= lr) ? dacc[r] : 0.f;
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J == I) Af[J] = dacc;
      else if (J > I) Af[J] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // -- off-diagonal sub-blocks J < I
#pragma unroll
    for (int J = 0; J < NB - 1; ++J) {
      if (J < I) {
        const int pr = I * (I - 1) / 2 + J;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float mm[8], x[8];
          lds8(&sM[pr][32 * ks + lk], mm);
#pragma unroll
          for (int c = 0; c < 8; ++c) x[c] = qt[8 * ks + c] * mm[c];
          const half8 ka = *reinterpret_cast<const half8*>(&sKt[16 * J + lr][32 * ks + lk]);
          acc = mfma16x16x32(ka, cvt8(x), acc);
        }
        Af[J] = acc;
      }
    }
    // -- entries beyond 2^14 (large q and k): divide the wave's blocks by a
    // power of two, undone on the accumulators
    float am = 0.f;
#pragma unroll
    for (int J = 0; J < NB; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(Af[J][r]));
    if (__any(am > kRowRange)) {
      sigA = uniform(row_scale(group_max<64>(am)));
      const float inv = inv_scale(sigA);
#pragma unroll
      for (int J = 0; J < NB; ++J) Af[J] *= inv;
    }
#pragma unroll
    for (int J = 0; J < NB; ++J) A[J] = cvt4(Af[J]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float eb[8], x[8];
      lds8(&sEb[I][32 * ks + lk], eb);
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = qt[8 * ks + c] * eb[c];
      qh[ks] = cvt8(x);
    }
  }

  // O_I = sum_{J<=I} A_IJ V_J on the matrix cores (single pass and runs)
  auto intra_av = [&](floatx4 (&oacc)[NE]) {
#pragma unroll
    for (int E = 0; E < NE; ++E) {
      oacc[E] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (owner) {
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            oacc[E] = mfma16x16x16(vb, A[J], oacc[E]);
          }
        }
      }
    }
  };
  if constexpr (!kFused) {
    __syncthreads();  // K~ is no longer read: its LDS becomes the output tile
    // -- O_I = sum_{J<=I} A_IJ V_J + Q^_I S, with A stored / sigA and the
    // readout taken / max sigS
    if (owner) {
      const float smax = uniform(sSigMax);
      const bool rescale = sigA != 1.f || smax != 1.f;
      const float f1 = sigA * inv_scale(smax);
#pragma unroll
      for (int E = 0; E < NE; ++E) {
        // one accumulation chain of a single product shape (16x16x16) per value
        // block: the readout contracts four key dims per lane group per step
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            acc = mfma16x16x16(vb, A[J], acc);
          }
        }
        if (rescale) acc *= f1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb = ld_tr<SSTR, 8>(&sS[32 * ks + 4 * hh][16 * E]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            acc = mfma16x16x16(sb, qa, acc);
          }
        }
        if (rescale) acc *= smax;
        stage_out(acc, E);
      }
    }
  } else {
    float xs[NGR][8];  // S_n, by groups of 8 elements of one state row
    floatx4 oacc[NE];  // the outputs, O_I
    if constexpr (GR == 1) {
    // -- the entering state, in-segment part: X and W
    const int seg = n / G, n0 = seg * G, nlast = min(n0 + G, N) - 1;
    const bool agg = n == nlast && seg < nseg - 1;  // publishes the segment's aggregate
    if (wave == 0) wave_wait_flags(cw + n0, n - n0, ctrl);
    __syncthreads();
    float wv[NGR];
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      wv[g] = 1.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) xs[g][c] = 0.f;
    }
    // all groups' loads of a batch of predecessors go out together
    for (int m = n - 1; m >= n0; m -= LB) {
      half8 u[NGR][LB];
      float a[NGR][LB], su[NGR][LB];
#pragma unroll
      for (int g = 0; g < NGR; ++g) {  // clamped, unconditional loads
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const int mj = m - j >= n0 ? m - j : n0;
          u[g][j] = ld_coh(rU, mj * DKDV + x8);
          const float2 p = ld_dev2(Aws + 2 * ((bh * N + mj) * DK + x8 / DV));  // (a, sigU)
          a[g][j] = p.x, su[g][j] = p.y;
        }
      }
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          if (x8 < DKDV && m - j >= n0) {
            const float w = wv[g] * su[g][j];
#pragma unroll
            for (int c = 0; c < 8; ++c) xs[g][c] += w * (float)u[g][j][c];
            wv[g] *= a[g][j];
          }
          consume(u[g][j], a[g][j]);
          consume(u[g][j], su[g][j]);
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
          const half8 un = *reinterpret_cast<const half8*>(&sU[d][x8 % DV]);  // own U_n
          float ag[8], m = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            ag[c] = sAn[d] * xs[g][c] + sSigU[d] * (float)un[c];
            m = fmaxf(m, fabsf(ag[c]));
          }
          // the DV/8 neighbouring lanes of row d agree on its scale
          float sg = 1.f;
          if (__any(m >= kRowRange)) {
            sg = row_scale(DV == 64 ? group_max<8>(m) : group_max<4>(m));
            const float inv = inv_scale(sg);
#pragma unroll
            for (int c = 0; c < 8; ++c) ag[c] *= inv;
          }
          st_coh(rS, seg * DKDV + x8, cvt8(ag));
          // with the segment's decay: the weight the look-back accumulated, times a_n
          if (x8 % DV == 0) st_dev2(GAws + 2 * (gs * DK + d), wv[g] * sAn[d], sg);
        }
      }
    }
    // -- intra-chunk part, while the aggregate's stores complete and the
    // earlier segments publish: O_I = sum_{J<=I} A_IJ V_J
    intra_av(oacc);
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
      float a[NGR][LB], su[NGR][LB];
#pragma unroll
      for (int g = 0; g < NGR; ++g) {  // clamped, unconditional loads
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const int sj = s2 - j >= 0 ? s2 - j : 0;
          u[g][j] = ld_coh(rS, sj * DKDV + x8);
          const float2 p = ld_dev2(GAws + 2 * ((bh * nseg + sj) * DK + x8 / DV));  // (decay, sig)
          a[g][j] = p.x, su[g][j] = p.y;
        }
      }
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          if (x8 < DKDV && s2 - j >= 0) {
            const float w = w2[g] * su[g][j];
#pragma unroll
            for (int c = 0; c < 8; ++c) pv[g][c] += w * (float)u[g][j][c];
            w2[g] *= a[g][j];
          }
          consume(u[g][j], a[g][j]);
          consume(u[g][j], su[g][j]);
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
          load_f8(s0 + st_at(x8 / DV, x8 % DV), z);
#pragma unroll
          for (int c = 0; c < 8; ++c) pv[g][c] += w2[g] * z[c];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[g][c] += wv[g] * pv[g][c];  // S_n
        if (fin) {
          float f[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) f[c] = sAn[d] * xs[g][c] + sSigU[d] * (float)ul[g][c];
          store_f8(sfin + st_at(x8 / DV, x8 % DV), f);
        }
      }
    }
    } else {
      // -- runs: the intra-chunk part first, O_I = sum_{J<=I} A_IJ V_J
      intra_av(oacc);
      // -- the state entering the run, S_in: its predecessors' aggregates
      // folded onto the nearest inclusive state (or the initial state)
      int nagg = 0, from_start = 1;
      if (run > 0) {
        if (threadIdx.x < 64) {
          int fs;
          const int na = lookback_runs(cw, run, ctrl, &fs);
          if (threadIdx.x == 0) sLook[0] = na, sLook[1] = fs;
        }
        __syncthreads();
        nagg = sLook[0], from_start = sLook[1];
      }
      float pv[NGR][8], w2[NGR];
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        w2[g] = 1.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) pv[g][c] = 0.f;
      }
      for (int j = 0; j < nagg; j += LB) {
        half8 u[NGR][LB];
        float a[NGR][LB], su[NGR][LB];
#pragma unroll
        for (int g = 0; g < NGR; ++g) {  // clamped, unconditional loads
          const int x8 = (8 * (tid + kThreads * g)) % DKDV;
#pragma unroll
          for (int jj = 0; jj < LB; ++jj) {
            const int r = run - 1 - min(j + jj, nagg - 1);
            u[g][jj] = ld_coh(rU, r * DKDV + x8);
            const float2 pr = ld_dev2(Aws + 2 * ((bh * nseg + r) * DK + x8 / DV));  // (decay, sig)
            a[g][jj] = pr.x, su[g][jj] = pr.y;
          }
        }
#pragma unroll
        for (int g = 0; g < NGR; ++g) {
#pragma unroll
          for (int jj = 0; jj < LB; ++jj) {
            if (j + jj < nagg) {
              const float w = w2[g] * su[g][jj];
#pragma unroll
              for (int c = 0; c < 8; ++c) pv[g][c] += w * (float)u[g][jj][c];
              w2[g] *= a[g][jj];
            }
            consume(u[g][jj], a[g][jj]);
            consume(u[g][jj], su[g][jj]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = (8 * (tid + kThreads * g)) % DKDV;
        if (!from_start) {
          const int r = run - 1 - nagg;
          const half8 u = ld_coh(rS, r * DKDV + x8);
          const float w = w2[g] * ld_dev2(GAws + 2 * ((bh * nseg + r) * DK + x8 / DV)).y;
#pragma unroll
          for (int c = 0; c < 8; ++c) pv[g][c] += w * (float)u[c];
        } else if (s0) {
          float z[8];
          load_f8(s0 + st_at(x8 / DV, x8 % DV), z);
#pragma unroll
          for (int c = 0; c < 8; ++c) pv[g][c] += w2[g] * z[c];
        }
      }
      // -- this chunk's state S_n = X + W S_in, X and W from the run's chunks
      // before it; the run's last chunk also forms a_n S_n + U_n, the run's
      // inclusive state (published for the later runs) or the final state
      const bool last_run = run == nseg - 1;
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
        float x[8], w;
        run_prefix(grp, x8 % DKDV, x, w);
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[g][c] = fmaf(w, pv[g][c], x[c]);
        if (grp == GR - 1 && x8 < DKDV) {
          const half8 un = *reinterpret_cast<const half8*>(&sU[d][x8 % DV]);
          float inc[8], m = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            inc[c] = fmaf(sSigU[d], (float)un[c], sAn[d] * xs[g][c]);
            m = fmaxf(m, fabsf(inc[c]));
          }
          if (last_run) {
            if (sfin) store_f8(sfin + st_at(x8 / DV, x8 % DV), inc);
          } else {
            const float sg = row_scale(DV == 64 ? group_max<8>(m) : group_max<4>(m));
            const float inv = inv_scale(sg);
#pragma unroll
            for (int c = 0; c < 8; ++c) inc[c] *= inv;
            st_coh(rS, run * DKDV + x8, cvt8(inc));
            if (x8 % DV == 0) st_dev2(GAws + 2 * ((bh * nseg + run) * DK + d), 1.f, sg);
          }
        }
      }
      __syncthreads();  // every U tile read: the region becomes S_n's staging tile
      if (grp == GR - 1 && !last_run) publish_wave(cw + run, &sPub2, kStInc);
    }
    // -- S_n staged in half, row d divided by its scale
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      const int x8 = 8 * (tid + kThreads * g), d = x8 / DV;
      if (x8 < DKDV) {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(xs[g][c]));
        float o[8], sg = 1.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = xs[g][c];
        if (__any(m >= kRowRange)) {
          sg = row_scale(DV == 64 ? group_max<8>(m) : group_max<4>(m));
          const float inv = inv_scale(sg);
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c] *= inv;
          if (sg != 1.f) atomicMax(&sSigMaxBits, __float_as_uint(sg));  // positive floats
        }
        *reinterpret_cast<half8*>(&sS[d][x8 % DV]) = cvt8(o);
        if (x8 % DV == 0) sSig[d] = sg;
      }
    }
    __syncthreads();  // S_n complete in LDS; every read of published data done
    // -- readout, on the same accumulation chains: O_I += Q^_I S_n, with the
    // row scales of S_n folded into Q^ (factors sigS[d] / max sigS <= 1) and
    // the accumulators taken / max sigS meanwhile
    if (owner) {
      // the largest row scale (1 unless some row was scaled)
      const float smax = uniform(__uint_as_float(sSigMaxBits));
      if (smax != 1.f) {
        const float is = inv_scale(smax);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float f[8], x[8];
          lds8(&sSig[32 * ks + lk], f);
#pragma unroll
          for (int c = 0; c < 8; ++c) x[c] = (float)qh[ks][c] * (f[c] * is);
          qh[ks] = cvt8(x);
        }
      }
      const bool rescale = sigA != 1.f || smax != 1.f;
      const float f1 = sigA * inv_scale(smax);
#pragma unroll
      for (int E = 0; E < NE; ++E) {
        if (rescale) oacc[E] *= f1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb = ld_tr<SSTR, 8>(&sS[32 * ks + 4 * hh][16 * E]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            oacc[E] = mfma16x16x16(sb, qa, oacc[E]);
          }
        }
        if (smax != 1.f) oacc[E] *= smax;
        stage_out(oacc[E], E);
      }
    }
  }
  __syncthreads();

  // -- scatter rows back to their raster positions; with the output gate,
  // each row of dv values becomes o / sqrt(mean(o^2) + eps) * w * silu(z)
  // (its dv/8 lanes are neighbours and reduce the sum of squares by shuffles)
  constexpr int LPR = DV / 8;  // lanes per output row
  for (int u = tid; u < C * LPR; u += kThreads) {
    const int r = u / LPR, c8 = (u % LPR) * 8;
    const long orow = (((long)b * T + (sRow[r] >= 0 ? sRow[r] : 0)) * H + hr) * VP + vs * DV;
    if constexpr (!kGate) {
      if (sRow[r] >= 0) out8(op + orow + c8, &sO[r][c8]);
      continue;
    }
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = (float)sO[r][c8 + c];
    if constexpr (kGate) {
      float z[8], wn[8];
      load8(zp + orow + c8, z);
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
    if (sRow[r] >= 0) out8(op + orow + c8, x);
  }
  if constexpr (kFused && GR == 1) {
    // -- this chunk is done reading what its chain published: count it; the
    // last chunk of the chain to finish clears the chain's control words (off
    // the critical path, after the outputs are on their way)
    if (tid == 0) sDone = atomicAdd(ctrl + kCtrlHeader + bh * (long)(N + nseg + 1) + N + nseg, 1u);
    __syncthreads();
    if (sDone == (unsigned)(N - 1)) {
      unsigned* cw = ctrl + kCtrlHeader + bh * (long)(N + nseg + 1);
      for (int i = tid; i < N + nseg + 1; i += kThreads) cw[i] = 0u;
    }
  } else if constexpr (kFused) {
    // -- runs: the same per run (status words, then the counter)
    unsigned* cw = ctrl + kCtrlHeader + bh * (long)(nseg + 1);
    if (threadIdx.x == 0) sLook[0] = (int)atomicAdd(cw + nseg, 1u);
    __syncthreads();
    if (sLook[0] == nseg - 1)
      for (int i = threadIdx.x; i < nseg + 1; i += kThreads * GR) cw[i] = 0u;
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
                     reinterpret_cast<const float*>(ws + w.off_ss) + bhn * DK,
                     nullptr, nullptr, nullptr, nullptr,
                     kGate ? static_cast<const InT*>(epi.gate) + tok * DV : nullptr,
                     epi.weight, epi.eps, p.T, p.H, p.N, 1, 1, p.gh, p.gw, dirs);
  return hipGetLastError();
}

// One single-pass launch of chunk_kernel with DVW value columns per
// workgroup and VS = DV / DVW workgroups per chunk-head (the workspace
// arrays are indexed by the B x H VS chains; U tiles and states keep their
// size, the (decay, scale) pairs are VS times as many)
template <int DK, int DV, int DVW, int C, typename InT, bool kGate>
hipError_t onepass_launch(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                          const void* k, const void* v, const void* gk, void* o, char* ws,
                          const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  constexpr int VS = DV / DVW;
  const WsLayout w = workspace_layout(p);
  const Segments sg = onepass_segments(p.N);
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * VS * p.N;
  const long bhs = (long)b0 * p.H * VS * sg.nseg;
  const long st = (long)b0 * p.H * DK * DV;
  // chunk-major: chunk n of every (batch, head) chain before chunk n + 1
  dim3 grid((unsigned)((long)nb * p.H * VS * p.N));
  hipLaunchKernelGGL((chunk_kernel<DK, DVW, C, InT, true, kGate, 1, VS>), grid, dim3(kThreads), 0, s,
                     static_cast<const InT*>(q) + tok * DK, static_cast<const InT*>(k) + tok * DK,
                     static_cast<const InT*>(v) + tok * DV, static_cast<const InT*>(gk) + tok * DK,
                     static_cast<InT*>(o) + tok * DV,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhn * DK * DVW,
                     reinterpret_cast<float*>(ws + w.off_a) + 2 * bhn * DK,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhs * DK * DVW, nullptr,
                     reinterpret_cast<float*>(ws + w.off_g) + 2 * bhs * DK,
                     reinterpret_cast<unsigned*>(ws), s0 ? s0 + st : nullptr,
                     sfin ? sfin + st : nullptr,
                     kGate ? static_cast<const InT*>(epi.gate) + tok * DV : nullptr, epi.weight,
                     epi.eps, p.T, p.H, p.N, sg.G, sg.nseg, p.gh, p.gw, dirs);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename InT, bool kGate>
hipError_t onepass_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                     const void* k, const void* v, const void* gk, void* o, char* ws,
                     const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  if constexpr (DV == 64 && !kGate) {
    if (p.vs == 2)
      return onepass_launch<DK, DV, DV / 2, C, InT, kGate>(p, b0, nb, dirs, q, k, v, gk, o, ws,
                                                           s0, sfin, epi, s);
  }
  if (p.vs != 1) return hipErrorInvalidValue;
  return onepass_launch<DK, DV, DV, C, InT, kGate>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin,
                                                   epi, s);
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
