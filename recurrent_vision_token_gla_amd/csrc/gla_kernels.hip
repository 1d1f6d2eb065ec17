// gfx950 kernels of the chunkwise key-only GLA forward.
//
// Schedule (GTR project page, "A Kernel That Makes Recurrence Fast"; ai.info
// summary of GTR, "Methodology in Plain English"): per-chunk summaries in
// parallel over the chunk x head grid, a light scan of the chunk-boundary
// states along the chunk axis, then every chunk's outputs in parallel with the
// causal intra-chunk tile held on chip (in registers) and the boundary-state
// readout fused in. All three phases read their tokens through the scan-order index
// math, so no permuted copy of any tensor is ever made.
//
// Notation inside a chunk of C tokens (local index i), per key dim d, with
// g2 = gk * log2(e) so that every exponential is a base-2 exp2:
//   b_i = sum_{r<=i} g2_r                 inclusive cumulative log2-decay
//   B   = b_{C-1}                          (padding tokens have g2 = 0)
// Every decay factor fed to a half-precision matrix product off the score
// tile's diagonal is <= 1 in magnitude (times |q| or |k|), so strong decay
// cannot overflow it:
//   summary : K^[j] = k_j * 2^(B - b_j)
//   readout : Q^[i] = q_i * 2^(b_i)
//   off-diagonal 16x16 sub-blocks (I > J) of the score tile:
//       Q~[i] = q_i 2^(b_i - beta_I),  K~[j] = k_j 2^(e_J - b_j),
//       m_IJ  = 2^(beta_I - e_J)
//     with beta_I = b at the token before sub-block I and e_J = b at the
//     last token of sub-block J; A_IJ = (Q~_I * m_IJ) K~_J^T.
//   diagonal sub-blocks: one reference at the sub-block's 8th token,
//     q_i 2^(b_i - b_7) and k_j 2^(b_7 - b_j), factors up to 2^range; each
//     wave picks half operands, float operands or a direct sum of every entry
//     from the range and the operands' magnitude (chunk_kernel).
// Stored states (U, S, aggregates) are half rows divided by power-of-two
// row scales (row_scale in gla_tile.h), so any state fp32 holds fits.
#include "gla_launch.h"

#include "gla_chunk.h"

namespace gla {
namespace tile {

// ===========================================================================
// Phase 1: chunk summaries. One workgroup per (chunk n, head h, batch b).
//   U[d][e] = sum_j K^[j][d] V[j][e],     K^[j] = k_j 2^(B - b_j)  (<= |k|)
//   a[d]      = 2^(B[d]), stored as the pair (a[d], m[d]) with m[d] the
//               largest |U[d][e]| (the scan's bound needs it; U's row scale
//               is row_scale(m[d]))
// Wave w owns the 16 tokens of sub-block w, one token per lane row, and
// takes its cumulative decay with a DPP row scan plus the totals of the
// earlier sub-blocks. K^ and V go to LDS as token rows (16-byte stores) and
// both operands of the token contraction come back through the transposing
// LDS read; U is produced (as U^T) in 16x16 blocks on the matrix cores,
// staged through LDS as rows of key dims and stored as half [dk][dv], each
// row d divided by its power-of-two scale sigU[d] (row_scale of the row's
// largest magnitude, taken exactly through LDS).
// ===========================================================================
template <int DK, int DV, int C, typename InT>
__global__ __launch_bounds__(kThreads, 7) void summary_kernel(
    const InT* __restrict__ kp, const InT* __restrict__ vp, const InT* __restrict__ gp,
    half_t* __restrict__ Uws, float* __restrict__ Aws, int T, int H, int N, int gh, int gw,
    DirPack dirs) {
  constexpr int NB = C / 16, NKS = DK / 32, NEL = 8 * NKS, NE = DV / 16, ND = DK / 16;
  constexpr int VSTR = DV + 16;  // halves, rows of V (read transposed)
  constexpr int HSTR = DK + 16;  // halves, rows of K^ (read transposed)
  constexpr int USTR = DV + 8;   // halves, staging rows of U (one row per key dim)
  // the U staging tile reuses K^'s LDS once the products have read it
  constexpr int KU_BYTES = (C * HSTR > DK * USTR ? C * HSTR : DK * USTR) * 2;
  __shared__ __attribute__((aligned(16))) half_t sV[C][VSTR];
  __shared__ __attribute__((aligned(16))) char sKU[KU_BYTES];
  __shared__ __attribute__((aligned(16))) float sTot[NB][DK];
  __shared__ __attribute__((aligned(16))) float sAft[NB][DK];  // totals of sub-blocks I..NB-1
  __shared__ unsigned sRowMax[DK];  // largest |U[d][e]| of each row, as float bits
  half_t (*sKh)[HSTR] = reinterpret_cast<half_t (*)[HSTR]>(sKU);
  half_t (*sU)[USTR] = reinterpret_cast<half_t (*)[USTR]>(sKU);

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = 8 * lq;
  const int dir = dirs.get(b);

  const bool owner = wave < NB;
  const int I = wave, t = 16 * I + lr;
  RawRow<InT, NKS> kr, gr;  // as loaded, converted where consumed
  float sc[NEL];
  bool pad;  // this lane's token row is padding
  {
    const int rr = owner ? token_row(n * C + t, T, gh, gw, dir) : -1;
    const long row = rr >= 0 ? ((long)b * T + rr) * H + h : -1;
    pad = row < 0;
    kr.load(kp, row, DK, lk);
    gr.load(gp, row, DK, lk);
  }
  // V rows: written to LDS after the decay scan (float inputs: at once,
  // they have no registers to spare)
  VRows<DV, C, VSTR, InT> vrows;
  vrows.load(vp, n * C, T, gh, gw, dir, (long)b * T, H, h, DV, threadIdx.x);
  if constexpr (sizeof(InT) == 4) vrows.store(n * C, T, sV, threadIdx.x);
  if (tid < DK) sRowMax[tid] = 0u;
  if ((n + 1) * C > T) {  // the chain's last chunk: zero the padding rows
    kr.zero_if(pad);
    gr.zero_if(pad);
  }
  if (owner) {
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(mulw(gr[e], kLog2e));
    if (lr == 15) {
#pragma unroll
      for (int e = 0; e < NEL; ++e) sTot[I][32 * (e / 8) + lk + (e % 8)] = sc[e];
    }
  }
  if constexpr (sizeof(InT) == 2) vrows.store(n * C, T, sV, threadIdx.x);
  __syncthreads();

  const long bhn = ((long)b * H + h) * N + n;
  if (tid < NB * DK) {
    const int I2 = tid / DK, d = tid % DK;
    float aft = 0.f;
    for (int J = I2; J < NB; ++J) aft += sTot[J][d];
    sAft[I2][d] = aft;
  }
  __syncthreads();
  if (owner) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float aft[8];
      lds8(&sAft[I][32 * ks + lk], aft);
      half8 kh8;
#pragma unroll
      for (int c = 0; c < 8; ++c)  // B - b_t: the decay of the later tokens
        kh8[c] = (half_t)mulw(kr[8 * ks + c], fexp2(aft[c] - sc[8 * ks + c]));
      *reinterpret_cast<half8*>(&sKh[t][32 * ks + lk]) = kh8;
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
        const half4 a = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
        const half4 bb = ld_tr<HSTR, 4>(&sKh[16 * J][16 * D]);
        acc[i] = mfma16x16x16(a, bb, acc[i]);
      }
      // this lane's four values of row d = 16D + lr
      const float m = fmaxf(fmaxf(fabsf(acc[i][0]), fabsf(acc[i][1])),
                            fmaxf(fabsf(acc[i][2]), fabsf(acc[i][3])));
      atomicMax(&sRowMax[16 * D + lr], __float_as_uint(m));
    }
  }
  __syncthreads();  // K^ is no longer read; the row maxima are complete
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + 4 * i;
    if (blk < NBLK) {
      const int E = blk / ND, D = blk % ND;
      const float inv = inv_scale(row_scale(__uint_as_float(sRowMax[16 * D + lr])));
      const floatx4 x = acc[i] * inv;
      *reinterpret_cast<half4*>(&sU[16 * D + lr][16 * E + 4 * lq]) = cvt4(x);
    }
  }
  __syncthreads();
  half_t* Ub = Uws + bhn * (long)(DV * DK);
  for (int u = tid; u < DK * (DV / 8); u += kThreads) {
    const int d = u / (DV / 8), e8 = (u % (DV / 8)) * 8;
    *reinterpret_cast<half8*>(Ub + d * DV + e8) = *reinterpret_cast<const half8*>(&sU[d][e8]);
  }
  if (tid < DK)  // (a = 2^B, largest |U| of row d)
    *reinterpret_cast<float2*>(Aws + 2 * (bhn * DK + tid)) =
        float2{fexp2(sAft[0][tid]), __uint_as_float(sRowMax[tid])};
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
// The serial scan below replaces the segmented one from this many state
// element groups of 8 per launch (B H dk dv / 8), or from half as many for
// chains of 256 chunks and more. Measured on MI355X (64/64, each scan alone,
// 20 launches captured in one graph, segmented / serial, us; the serial scan
// with its window refilled in halves and four elements per thread):
//   groups   N=25          N=100          N=256
//    8,192   4.3 / 5.6     9.2 / 15.7     26.2 / 33.5
//   16,384   5.7 / 6.0    15.0 / 16.4      - / 33.6 (segmented 38.3 earlier)
//   32,768    - / 6.6       - / 17.9     (segmented 7.4 and 22.3 earlier)
constexpr long kSerialScanGroups = 32768;
constexpr int kSerialScanLongChain = 256;

// R: chunks per segment kept in registers (2, 4 or 8, the segment length
// rounded up, so that the clamped loads of a short segment are not repeated)
//
// Scales: U_n arrives as half rows divided by row_scale(m_n[d]), m_n[d] its
// largest magnitude (paired with a_n[d] in one 8-byte load). S_n leaves as
// half rows divided by row_scale(M_n[d]), with M_n[d] a bound on
// max_e |S_n[d][e]| that every thread of a row computes identically:
//   M_0 = max_e |s0[d][e]|,   M_{n+1} = a_n M_n + m_n[d],
// so the stored rows stay below 2^14 and no row maximum has to be exchanged
// on the way. The bound composes over segments like (a, U) does. The scales
// are taken from exponents (v_ldexp) without branches: a branch on freshly
// loaded data would make the compiler wait for every load in flight.
template <int kScanRegs>
__global__ __launch_bounds__(kThreads) void scan_kernel(
    const half_t* __restrict__ Uws, const float* __restrict__ Aws, half_t* __restrict__ Sws,
    float* __restrict__ SigS, const float* s0, float* sfin, int H, int N, int DK, int DV, int L) {
  __shared__ unsigned sM0[8 * (kThreads / kScanSegs) / 32];  // per state row of the block
  const long bh = (long)blockIdx.z * H + blockIdx.y;
  const int seg = threadIdx.x & (kScanSegs - 1);
  const int x8 = 8 * (blockIdx.x * (kThreads / kScanSegs) + (threadIdx.x >> 4));
  const int d = x8 / DV;
  const long DKDV = (long)DK * DV;
  const half_t* U = Uws + bh * N * DKDV + x8;
  const float2* A = reinterpret_cast<const float2*>(Aws) + bh * N * DK + d;  // (a, m)
  half_t* S = Sws + bh * N * DKDV + x8;
  float* SS = SigS + bh * N * DK + d;
  const bool row_lead = x8 % DV == 0;  // this group stores its row's scale
  const int n0 = min(seg * L, N), n1 = min(n0 + L, N);

  // -- fold this segment into (ag, ug) and its bound mg; the chunks of one
  // register block stay cached
  float ag = 1.f, mg = 0.f, ug[8];
  half8 uc[kScanRegs];
  float2 ac[kScanRegs];
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
        const float su = __builtin_amdgcn_ldexpf(1.f, row_scale_exp(ac[i].y));
#pragma unroll
        for (int c = 0; c < 8; ++c) ug[c] = fmaf((float)uc[i][c], su, ac[i].x * ug[c]);
        mg = ac[i].x * mg + ac[i].y;
        ag *= ac[i].x;
      }
    }
  }
  // -- inclusive composition over the segments of this row, then shift by one
#define GLA_SCAN_STEP(CTRL)                                              \
  {                                                                      \
    const float ap = dpp_row_shr<CTRL>(ag, 1.f);                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) ug[c] =                \
        ag * dpp_row_shr<CTRL>(ug[c], 0.f) + ug[c];                      \
    mg = ag * dpp_row_shr<CTRL>(mg, 0.f) + mg;                           \
    ag *= ap;                                                            \
  }
  GLA_SCAN_STEP(0x111)
  GLA_SCAN_STEP(0x112)
  GLA_SCAN_STEP(0x114)
  GLA_SCAN_STEP(0x118)
#undef GLA_SCAN_STEP
  float st0[8], s[8], M0 = 0.f;
  if (s0) {  // uniform: the initial state and its row maxima (rows span two waves)
    if (threadIdx.x < 8 * (kThreads / kScanSegs) / 32) sM0[threadIdx.x] = 0u;
    load_f8(s0 + bh * DKDV + x8, st0);
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(st0[c]));
    __syncthreads();
    atomicMax(&sM0[(8 * (threadIdx.x >> 4)) / DV], __float_as_uint(m));
    __syncthreads();
    M0 = __uint_as_float(sM0[(8 * (threadIdx.x >> 4)) / DV]);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) st0[c] = 0.f;
  }
  const float ae = dpp_row_shr<0x111>(ag, 1.f);
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = ae * st0[c] + dpp_row_shr<0x111>(ug[c], 0.f);
  float M = ae * M0 + dpp_row_shr<0x111>(mg, 0.f);
  if (sfin && seg == kScanSegs - 1) {
    float f[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) f[c] = ag * st0[c] + ug[c];
    store_f8(sfin + bh * DKDV + x8, f);
  }
  // -- replay the segment from its entering state; a segment longer than one
  // register block reads its chunks again (the registers hold the last
  // block). The state is kept divided by its current row scale 2^es, which
  // the update folds in (exact power-of-two factors), so each stored row is
  // a plain conversion.
  int es = row_scale_exp(M);
  {
    const float inv = __builtin_amdgcn_ldexpf(1.f, -es);
#pragma unroll
    for (int c = 0; c < 8; ++c) s[c] *= inv;
  }
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
        half8 o;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = (half_t)s[c];
        *reinterpret_cast<half8*>(S + (long)(nb + i) * DKDV) = o;
        if (row_lead) SS[(long)(nb + i) * DK] = __builtin_amdgcn_ldexpf(1.f, es);
        M = ac[i].x * M + ac[i].y;
        const int en = row_scale_exp(M);
        // s <- (a s + sigU u) / 2^en, with s held / 2^es (the factors are
        // powers of two, so this is exact scaling of the unscaled update; no
        // branch: one on loaded data would wait for every load in flight)
        const float f = __builtin_amdgcn_ldexpf(ac[i].x, es - en);
        const float g = __builtin_amdgcn_ldexpf(1.f, row_scale_exp(ac[i].y) - en);
#pragma unroll
        for (int c = 0; c < 8; ++c) s[c] = fmaf((float)uc[i][c], g, f * s[c]);
        es = en;
      }
    }
  }
}

// The boundary scan for many chains at once: one thread per state element
// group of EPT (4 or 8), walking its chain's chunks in order with the loads
// of the next W/2 to W chunks in flight. A wave's load of one chunk covers
// 64 EPT contiguous halves of state (the segmented scan above touches 16
// chunks in 64-byte pieces per load and makes two dependent memory round
// trips per workgroup); with
// enough chains the loads in flight cover the HBM latency, and each element
// follows the recurrence S_{n+1} = a_n S_n + U_n exactly in order. Scales as
// in scan_kernel; the DV/EPT threads of a state row are neighbouring lanes,
// which take the row maximum of s0 by lane permutations.
template <int W, int EPT>
__global__ __launch_bounds__(kThreads) void scan_serial_kernel(
    const half_t* __restrict__ Uws, const float* __restrict__ Aws, half_t* __restrict__ Sws,
    float* __restrict__ SigS, const float* s0, float* sfin, int N, int DK, int DV, long groups) {
  typedef _Float16 HV __attribute__((ext_vector_type(EPT)));
  typedef float FV __attribute__((ext_vector_type(EPT)));
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  // groups is a multiple of DV/EPT, so the lanes of one state row leave together
  if (gid >= groups) return;
  const long DKDV = (long)DK * DV, per = DKDV / EPT;
  const long bh = gid / per;
  const int xg = EPT * (int)(gid - bh * per), d = xg / DV;
  const half_t* U = Uws + bh * N * DKDV + xg;
  const float2* A = reinterpret_cast<const float2*>(Aws) + bh * N * DK + d;  // (a, m)
  half_t* S = Sws + bh * N * DKDV + xg;
  float* SS = SigS + bh * N * DK + d;
  const bool row_lead = xg % DV == 0;
  float s[EPT], M = 0.f;
  if (s0) {
    const FV x = *reinterpret_cast<const FV*>(s0 + bh * DKDV + xg);
#pragma unroll
    for (int c = 0; c < EPT; ++c) s[c] = x[c], M = fmaxf(M, fabsf(s[c]));
    if constexpr (EPT == 8) M = DV == 64 ? group_max<8>(M) : group_max<4>(M);
    else M = DV == 64 ? group_max<16>(M) : group_max<8>(M);
  } else {
#pragma unroll
    for (int c = 0; c < EPT; ++c) s[c] = 0.f;
  }
  HV u[W];
  float2 a[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const long m = i < N ? i : N - 1;
    u[i] = *reinterpret_cast<const HV*>(U + m * DKDV);
    a[i] = A[m * DK];
  }
  // the state is kept divided by its current row scale 2^es (as in scan_kernel)
  int es = row_scale_exp(M);
  {
    const float inv = __builtin_amdgcn_ldexpf(1.f, -es);
#pragma unroll
    for (int c = 0; c < EPT; ++c) s[c] *= inv;
  }
  // chunk n from slot i (a constant once the loops below are unrolled)
  auto step = [&](int i, int n) {
    // the state entering chunk n
    HV o;
#pragma unroll
    for (int c = 0; c < EPT; ++c) o[c] = (half_t)s[c];
    *reinterpret_cast<HV*>(S + n * DKDV) = o;
    if (row_lead) SS[(long)n * DK] = __builtin_amdgcn_ldexpf(1.f, es);
    M = a[i].x * M + a[i].y;
    const int en = row_scale_exp(M);
    const float f = __builtin_amdgcn_ldexpf(a[i].x, es - en);
    const float g = __builtin_amdgcn_ldexpf(1.f, row_scale_exp(a[i].y) - en);
#pragma unroll
    for (int c = 0; c < EPT; ++c) s[c] = fmaf((float)u[i][c], g, f * s[c]);
    es = en;
  };
  // the window as two halves of W/2 chunks: each half is consumed in order
  // and then refilled at once (chunks W ahead, clamped) while the other
  // half's loads stay in flight. Whole windows run with no condition inside
  // and the last N % W chunks after them: with a condition per chunk, or a
  // slot refilled as soon as it is consumed, the compiler's wait placement
  // drained the whole window once per W chunks.
  constexpr int HW = W / 2;
  auto refill = [&](int h, int nb) {
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      const long m = nb + j < N ? nb + j : N - 1;
      u[h * HW + j] = *reinterpret_cast<const HV*>(U + m * DKDV);
      a[h * HW + j] = A[m * DK];
    }
  };
  int n0 = 0;
  for (; n0 + W <= N; n0 += W) {
#pragma unroll
    for (int j = 0; j < HW; ++j) step(j, n0 + j);
    __builtin_amdgcn_sched_barrier(0);
    refill(0, n0 + W);
#pragma unroll
    for (int j = 0; j < HW; ++j) step(HW + j, n0 + HW + j);
    __builtin_amdgcn_sched_barrier(0);
    refill(1, n0 + W + HW);
  }
#pragma unroll
  for (int i = 0; i < W - 1; ++i)
    if (n0 + i < N) step(i, n0 + i);
  if (sfin) {
    const float sc = __builtin_amdgcn_ldexpf(1.f, es);
    FV f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) f[c] = s[c] * sc;
    *reinterpret_cast<FV*>(sfin + bh * DKDV + xg) = f;
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
                     reinterpret_cast<float*>(ws + w.off_a) + 2 * bhn * DK, p.T, p.H, p.N, p.gh,
                     p.gw, dirs);
  return hipGetLastError();
}

__global__ void ctrl_clear_kernel(unsigned* ctrl) {
  for (int i = threadIdx.x; i < kCtrlWords; i += blockDim.x) ctrl[i] = 0u;
}

}  // namespace tile

using namespace tile;

WsLayout workspace_layout(const Problem& p) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t units = (size_t)p.B * p.H * p.N;
  WsLayout w;
  w.off_U = (size_t)kCtrlWords * sizeof(unsigned);
  w.off_a = w.off_U + up(units * p.dk * p.dv * sizeof(half_t));
  w.off_S = w.off_a + up(units * p.dk * 2 * sizeof(float) * (p.dv == 64 ? 2 : 1));
  w.off_g = w.off_S + up(units * p.dk * p.dv * sizeof(half_t));
  w.off_ss = w.off_g + up(units * p.dk * 2 * sizeof(float));
  w.total = w.off_ss + up(units * p.dk * sizeof(float));
  return w;
}

Segments onepass_segments(int N) {
  // short chains: one segment (each chunk reads its <= 7 predecessors, one
  // publication hop); longer ones: about sqrt(N) segments of sqrt(N) chunks
  if (N <= 8) return Segments{N, 1};
  int G = 1;
  while (G * G < N) ++G;
  return Segments{G, (N + G - 1) / G};
}

bool onepass_fits(const Problem& p, int nb) {
  const Segments sg = onepass_segments(p.N);
  if (sg.G > 64 || sg.nseg > 64) return false;  // one wave watches every flag it waits on
  const long chains = (long)nb * p.H * p.vs;
  const long words = kCtrlHeader + chains * (p.N + sg.nseg + 1);
  return words <= kCtrlWords && chains * p.N <= 0x7fffffffL;
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
  const long groups = (long)nb * p.H * (dkdv / 8);
  if (groups >= kSerialScanGroups || (groups >= kSerialScanGroups / 2 && p.N >= kSerialScanLongChain)) {
    // four state elements per thread: twice the waves of eight, and the
    // scan's issue, not its loads, is what bounds it
    constexpr int kEpt = 4;
    const long threads = groups * (8 / kEpt);
    auto serial = p.N >= 64 ? scan_serial_kernel<16, kEpt> : scan_serial_kernel<8, kEpt>;
    hipLaunchKernelGGL(serial, dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, s, reinterpret_cast<const half_t*>(ws + w.off_U) + bhn * dkdv,
                       reinterpret_cast<const float*>(ws + w.off_a) + 2 * bhn * p.dk,
                       reinterpret_cast<half_t*>(ws + w.off_S) + bhn * dkdv,
                       reinterpret_cast<float*>(ws + w.off_ss) + bhn * p.dk,
                       s0 ? s0 + st : nullptr, sfin ? sfin + st : nullptr, p.N, p.dk, p.dv,
                       threads);
    return hipGetLastError();
  }
  auto kernel = L <= 2 ? scan_kernel<2> : L <= 4 ? scan_kernel<4> : scan_kernel<8>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s,
                     reinterpret_cast<const half_t*>(ws + w.off_U) + bhn * dkdv,
                     reinterpret_cast<const float*>(ws + w.off_a) + 2 * bhn * p.dk,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhn * dkdv,
                     reinterpret_cast<float*>(ws + w.off_ss) + bhn * p.dk,
                     s0 ? s0 + st : nullptr, sfin ? sfin + st : nullptr, p.H, p.N, p.dk, p.dv,
                     L);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename InT>
hipError_t outputs_plain(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                         const void* k, const void* v, const void* gk, void* o, const char* ws,
                         const Epilogue& epi, hipStream_t s) {
  return outputs_t<DK, DV, C, InT, false>(p, b0, nb, dirs, q, k, v, gk, o, ws, epi, s);
}

template <int DK, int DV, int C, typename InT>
hipError_t onepass_plain(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                         const void* k, const void* v, const void* gk, void* o, char* ws,
                         const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  return onepass_t<DK, DV, C, InT, false>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, epi, s);
}

hipError_t launch_outputs(const Problem& p, int b0, int nb, const DirPack& dirs,
                          const void* q, const void* k, const void* v, const void* gk,
                          void* o, const char* ws, const Epilogue& epi, hipStream_t s) {
  if (epi.gate) return launch_outputs_gated(p, b0, nb, dirs, q, k, v, gk, o, ws, epi, s);
  GLA_DISPATCH(outputs_plain, p, b0, nb, dirs, q, k, v, gk, o, ws, epi, s);
}

hipError_t launch_onepass(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                          const void* k, const void* v, const void* gk, void* o, char* ws,
                          const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  if (epi.gate)
    return launch_onepass_gated(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, epi, s);
  GLA_DISPATCH(onepass_plain, p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, epi, s);
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
