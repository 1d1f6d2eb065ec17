// The forward in one kernel over runs of chunks, with a decoupled look-back
// between runs (GTR project page, "A Kernel That Makes Recurrence Fast": the
// chunkwise recurrence with its state carried only between chunk
// boundaries; here the carried quantity is the state entering each run of G
// chunks).
//
// One workgroup takes G consecutive chunks (a run) of one (batch, head)
// chain. Workgroups are numbered run-major (every chain's run 0, then every
// chain's run 1, ...), so a run's predecessors were dispatched earlier and
// have usually finished by the time it needs them. A workgroup walks its run
// twice:
//   pass A: each chunk's summary only (k, gk, v: decays, K^ = k 2^(B - b),
//           U = K^T V on the matrix cores), folded into the run's aggregate
//           X <- diag(a_n) X + U_n in matrix-core accumulators, and the run's
//           decay; it publishes the aggregate, takes the state entering the
//           run, S_in, from its predecessors, and publishes the inclusive
//           state A_run S_in + X;
//   pass B: each chunk in full with the state carried along the run in
//           float accumulators, S <- diag(a_n) S + U_n: scores, A V, the
//           readout Q^ S and the stores, as the three-phase output kernel
//           does with S from the boundary scan.
// So the state never leaves the workgroup inside a run, one launch replaces
// three, and per chunk HBM sees the forward's own bytes plus a quarter of the
// run's published and looked-back tiles (pass B's second read of k, gk, v
// follows pass A's by a few microseconds). The next chunk's inputs load
// while the current one is processed, pass B's first chunk's during the
// look-back.
//
// Look-back (Merrill and Garland's decoupled look-back, with 8 KB state
// tiles): every run has a status word, 1 once its aggregate is published, 2
// once its inclusive state is. A run reads the statuses of its predecessors
// (up to 64 at a time, one lane each) and waits until there is a nearest
// predecessor p with status 2 and every run between p and itself has status
// >= 1 (or every predecessor down to the chain's start has status >= 1); it
// then combines those aggregates and p's inclusive state (or the initial
// state). A run publishes its aggregate without waiting on anything, so the
// lowest-numbered unfinished workgroup never waits on an unfinished one: with
// in-order dispatch on every XCD the kernel cannot deadlock, whether or not
// its grid is co-resident. Every wait is bounded (kSpinLimit polls; running
// out sets the workspace's sticky error bit).
//
// Published tiles are half rows divided by power-of-two row scales; tiles and
// (decay, scale) pairs are written and read with device-coherent accesses
// (the single pass's protocol), status words with relaxed device-scope
// atomics after s_waitcnt on the stores. Each chain counts the runs that have
// finished reading; the last one clears the chain's words, so they are zero
// between calls.
#include "gla_launch.h"
#include "gla_tile.h"

namespace gla {
namespace tile {

constexpr unsigned kStAgg = 1u, kStInc = 2u;

// publish_wave with a given status value
__device__ __forceinline__ void publish_status(unsigned* word, unsigned value, unsigned* count) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0 && atomicAdd(count, 1u) == kThreads / 64 - 1)
    __hip_atomic_store(word, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Eight consecutive input elements as loaded (half: one 16-byte load; float:
// two), kept raw until the chunk that needs them is processed.
template <typename InT> struct Raw8;
template <> struct Raw8<half_t> {
  half8 v;
  __device__ __forceinline__ void load(const half_t* p) { v = *reinterpret_cast<const half8*>(p); }
  __device__ __forceinline__ void get(float* x) const {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = (float)v[c];
  }
  __device__ __forceinline__ half8 h() const { return v; }
};
template <> struct Raw8<float> {
  floatx4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const floatx4*>(p);
    b = *reinterpret_cast<const floatx4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* x) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = a[c], x[c + 4] = b[c];
  }
  __device__ __forceinline__ half8 h() const {
    half8 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = (half_t)a[c], r[c + 4] = (half_t)b[c];
    return r;
  }
};

template <int DK, int DV, int C, typename InT, int G>
__global__ __launch_bounds__(kThreads, 2) void runs_kernel(
    const InT* __restrict__ qp, const InT* __restrict__ kp, const InT* __restrict__ vp,
    const InT* __restrict__ gp, InT* __restrict__ op, half_t* __restrict__ AggT,
    float* __restrict__ AggP, half_t* __restrict__ IncT, float* __restrict__ IncP,
    unsigned* __restrict__ ctrl, const float* s0, float* sfin, int T, int H, int N, int NS,
    int nch, int gh, int gw, DirPack dirs) {
  constexpr int NB = C / 16, NKS = DK / 32, NEL = 8 * NKS, NE = DV / 16, ND = DK / 16;
  static_assert(NB == 4, "runs of 64-token chunks: one 16-token sub-block per wave");
  constexpr int NPAIR = NB * (NB - 1) / 2;
  constexpr int DKDV = DK * DV;
  constexpr int KSTR = DK + 8;   // halves, rows of K~ (read along key dims)
  constexpr int VSTR = DV + 16;  // halves, rows of V (read transposed)
  constexpr int HSTR = DK + 16;  // halves, rows of K^ (read transposed)
  constexpr int SSTR = DV + 16;  // halves, rows of the aggregate / S (read transposed)
  constexpr int OSTR = DV + 8;   // rows of the output staging tile
  constexpr int NBLK = NE * ND, BPW = (NBLK + 3) / 4;  // U blocks per wave
  constexpr int NGR = (DKDV / 8 + kThreads - 1) / kThreads;  // state groups of 8 per thread
  constexpr int LB = 4;  // look-back tiles per batch of loads
  constexpr float kHalfRange = 8.f, kF32Range = 120.f;
  constexpr bool kPrefetch = true;
  constexpr int KO0 = C * KSTR * 2, KO1 = C * OSTR * (int)sizeof(InT);
  // K^ (C x HSTR halves) and the aggregate / S tile (DK x SSTR halves) share
  // one region, which also carries S_in in float when it changes layout
  constexpr int KH_BYTES = C * HSTR * 2, XS_BYTES = DK * SSTR * 2;
  constexpr int BIG0 = KH_BYTES + XS_BYTES, BIG1 = DKDV * 4;
  __shared__ __attribute__((aligned(16))) char sKO[KO0 > KO1 ? KO0 : KO1];  // K~, then outputs
  __shared__ __attribute__((aligned(16))) half_t sV[C][VSTR];
  __shared__ __attribute__((aligned(16))) char sBig[BIG0 > BIG1 ? BIG0 : BIG1];
  __shared__ __attribute__((aligned(16))) float sTot[NB][DK], sS7[NB][DK];
  __shared__ __attribute__((aligned(16))) float sEb[NB][DK], sF[NB][DK];
  __shared__ __attribute__((aligned(16))) float sR1[NB][DK], sR2[NB][DK];
  __shared__ __attribute__((aligned(16))) float sM[NPAIR][DK];
  __shared__ __attribute__((aligned(16))) float sWl[DK], sAn[DK], sSig[DK];
  __shared__ unsigned sRowMax[DK];
  __shared__ int sLook[2];
  __shared__ unsigned sPub, sDone;
  half_t (*sKt)[KSTR] = reinterpret_cast<half_t (*)[KSTR]>(sKO);
  InT (*sO)[OSTR] = reinterpret_cast<InT (*)[OSTR]>(sKO);
  half_t (*sKh)[HSTR] = reinterpret_cast<half_t (*)[HSTR]>(sBig);
  half_t (*sXs)[SSTR] = reinterpret_cast<half_t (*)[SSTR]>(sBig + KH_BYTES);
  float (*sS32)[DV] = reinterpret_cast<float (*)[DV]>(sBig);

  const int run = blockIdx.x / nch, ch = blockIdx.x - run * nch;
  const int h = ch % H, b = ch / H;
  const long bh = (long)b * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4, lk = 8 * lq;
  const int I = wave, t = 16 * I + lr;
  const int dir = dirs.get(b);
  const int ng = min(G, N - run * G);  // chunks in this run
  unsigned* cw = ctrl + kCtrlHeader + (long)ch * (NS + 1);  // this chain's status words, counter
  // this lane's state row in the accumulator layout: d = 16 * (wave % ND) + lr
  const int drow = 16 * (wave % ND) + lr;

  // -- with kPrefetch the next chunk's inputs load while the current one is
  // processed (else each chunk loads its own at its start):
  // this wave's token rows of q (pass B only), k, gk in the operand layout
  // and this thread's share of V's rows, raw until used
  constexpr int NIT = (C * (DV / 8) + kThreads - 1) / kThreads;
  Raw8<InT> rq[NKS], rk[NKS], rg[NKS], rv[NIT];
  bool rpad, rvpad[NIT];
  auto issue = [&](int n, bool with_q) {
    const int rr = token_row(n * C + t, T, gh, gw, dir);
    rpad = rr < 0;
    const long row = ((long)b * T + (rr >= 0 ? rr : 0)) * H + h;  // padding reads row 0
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (with_q) rq[ks].load(qp + row * DK + 32 * ks + lk);
      rk[ks].load(kp + row * DK + 32 * ks + lk);
      rg[ks].load(gp + row * DK + 32 * ks + lk);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int u = tid + kThreads * it;
      const int r = (u / (DV / 8)) % C, c8 = (u % (DV / 8)) * 8;
      const int vr = token_row(n * C + r, T, gh, gw, dir);
      rvpad[it] = vr < 0;
      rv[it].load(vp + (((long)b * T + (vr >= 0 ? vr : 0)) * H + h) * DV + c8);
    }
  };
  // V rows of the current chunk to LDS (zero for padding rows)
  auto put_v = [&]() {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int u = tid + kThreads * it;
      const int r = u / (DV / 8), c8 = (u % (DV / 8)) * 8;
      if (u < C * (DV / 8)) {
        half8 x = rv[it].h();
        if (rvpad[it]) x = half8{};
        *reinterpret_cast<half8*>(&sV[r][c8]) = x;
      }
    }
  };
  // the largest |x| of this lane's accumulator-layout values into its row
  auto row_max_into_lds = [&](const floatx4* X) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      if (wave + 4 * i < NBLK) {
        const float m = fmaxf(fmaxf(fabsf(X[i][0]), fabsf(X[i][1])),
                              fmaxf(fabsf(X[i][2]), fabsf(X[i][3])));
        atomicMax(&sRowMax[drow], __float_as_uint(m));
      }
    }
  };
  // this lane's accumulator-layout values into sXs, rows divided by their scales
  auto stage_rows = [&](const floatx4* X) {
    const float inv = inv_scale(row_scale(__uint_as_float(sRowMax[drow])));
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      if (blk < NBLK) {
        const floatx4 x = X[i] * inv;
        *reinterpret_cast<half4*>(&sXs[drow][16 * (blk / ND) + 4 * lq]) = cvt4(x);
      }
    }
  };

  floatx4 X[BPW];  // pass A: the run's aggregate; pass B: the state S
#pragma unroll
  for (int i = 0; i < BPW; ++i) X[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (tid < DK) sWl[tid] = 0.f;
  if (tid == 0) sPub = 0u;
  if (kPrefetch) issue(run * G, false);

  // ===== pass A: the run's aggregate
#pragma nounroll
  for (int g = 0; g < ng; ++g) {
    const int tok0 = (run * G + g) * C;
    if (!kPrefetch) issue(run * G + g, false);
    float kf[NEL], sc[NEL];
    const bool pad = rpad;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      rk[ks].get(&kf[8 * ks]);
      rg[ks].get(&sc[8 * ks]);
    }
    put_v();
    if (kPrefetch) {
      if (g + 1 < ng) issue(run * G + g + 1, false);
      else issue(run * G, true);  // pass B's first chunk, during the look-back
    }
    if (tok0 + C > T) {
      zero_row<NEL>(pad, kf);
      zero_row<NEL>(pad, sc);
    }
#pragma unroll
    for (int e = 0; e < NEL; ++e) sc[e] = row_scan16(sc[e]) * kLog2e;
    if (lr == 15) {
#pragma unroll
      for (int e = 0; e < NEL; ++e) sTot[I][32 * (e / 8) + lk + (e % 8)] = sc[e];
    }
    __syncthreads();
    if (tid < NB * DK) {  // totals of sub-blocks I..NB-1, the chunk's decay
      const int I2 = tid / DK, d = tid % DK;
      float aft = 0.f;
#pragma unroll
      for (int J = 0; J < NB; ++J) aft += J >= I2 ? sTot[J][d] : 0.f;
      sF[I2][d] = aft;
      if (I2 == 0) {
        sAn[d] = fexp2(aft);
        sWl[d] += aft;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float aft[8], x[8];
      lds8(&sF[I][32 * ks + lk], aft);
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = kf[8 * ks + c] * fexp2(aft[c] - sc[8 * ks + c]);
      *reinterpret_cast<half8*>(&sKh[t][32 * ks + lk]) = cvt8(x);
    }
    __syncthreads();
    {
      const float an = sAn[drow];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int blk = wave + 4 * i;
        if (blk < NBLK) {
          const int E = blk / ND, D = blk % ND;
          X[i] *= an;
#pragma unroll
          for (int J = 0; J < NB; ++J) {
            const half4 a = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            const half4 bb = ld_tr<HSTR, 4>(&sKh[16 * J][16 * D]);
            X[i] = mfma16x16x16(a, bb, X[i]);
          }
        }
      }
    }
    __syncthreads();  // sV, sKh, sF, sAn free for the next chunk
  }

  // ===== the run's aggregate X, its decay 2^(W), and the state entering it
  if (tid < DK) sRowMax[tid] = 0u;
  __syncthreads();
  row_max_into_lds(X);
  __syncthreads();
  stage_rows(X);
  if (tid < DK) {
    sSig[tid] = row_scale(__uint_as_float(sRowMax[tid]));
    sAn[tid] = fexp2(sWl[tid]);  // the run's decay
  }
  __syncthreads();  // aggregate staged in sXs (rows / sSig), run decay in sAn

  const __amdgpu_buffer_rsrc_t rA = coh_rsrc(AggT + (long)ch * NS * DKDV, (long)NS * DKDV);
  const __amdgpu_buffer_rsrc_t rI = coh_rsrc(IncT + (long)ch * NS * DKDV, (long)NS * DKDV);
  float xs[NGR][8];  // the state entering the run (group layout: 8 elements of one row)
  if (run > 0) {
    // -- publish the aggregate
#pragma unroll
    for (int gr = 0; gr < NGR; ++gr) {
      const int x8 = 8 * (tid + kThreads * gr);
      if (x8 < DKDV)
        st_coh(rA, run * DKDV + x8, *reinterpret_cast<const half8*>(&sXs[x8 / DV][x8 % DV]));
    }
    if (tid < DK) st_dev2(AggP + 2 * (((long)ch * NS + run) * DK + tid), sAn[tid], sSig[tid]);
    publish_status(cw + run, kStAgg, &sPub);
    // -- look-back: wave 0 finds the nearest inclusive predecessor p (or the
    // chain's start) with every run between p and this one aggregated
    if (wave == 0) {
      int found = -1, base_s0 = 0;
      for (int j0 = 0; found < 0; j0 += 64) {
        const int cnt = min(64, run - j0);  // predecessors run-1-j0-lane, lane < cnt
        for (long it = 0;; ++it) {
          unsigned v = 0u;
          if (lane < cnt)
            v = __hip_atomic_load(cw + (run - 1 - j0 - lane), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
          const unsigned long long inc = __ballot(lane < cnt && v == kStInc);
          const unsigned long long none = __ballot(lane < cnt && v == 0u);
          if (inc) {
            const int jl = __builtin_ctzll(inc);
            if ((none & ((1ull << jl) - 1ull)) == 0ull) {
              found = j0 + jl;
              break;
            }
          } else if (none == 0ull) {
            if (j0 + cnt == run) {  // every predecessor aggregated: start from s0
              found = run;
              base_s0 = 1;
            }
            break;  // all aggregated: the next window
          }
          if (it >= kSpinLimit) {  // give up (results invalid, recorded)
            if (lane == 0) atomicOr(ctrl, kErrSpin);
            found = j0 + cnt;
            base_s0 = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (lane == 0) sLook[0] = found, sLook[1] = base_s0;
    }
    __syncthreads();
    const int nagg = sLook[0], base_s0 = sLook[1];
    // -- combine: S_in = sum_{j < nagg} (prod of later decays) Agg_{run-1-j}
    //              + (prod of the decays of those nagg runs) (Inc_p or s0)
    float w[NGR];
#pragma unroll
    for (int gr = 0; gr < NGR; ++gr) {
      w[gr] = 1.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) xs[gr][c] = 0.f;
    }
    for (int j = 0; j < nagg; j += LB) {
      half8 u[NGR][LB];
      float a[NGR][LB], su[NGR][LB];
#pragma unroll
      for (int gr = 0; gr < NGR; ++gr) {
        const int x8 = (8 * (tid + kThreads * gr)) % DKDV;
#pragma unroll
        for (int jj = 0; jj < LB; ++jj) {
          const int r = run - 1 - min(j + jj, nagg - 1);
          u[gr][jj] = ld_coh(rA, r * DKDV + x8);
          const float2 pr = ld_dev2(AggP + 2 * (((long)ch * NS + r) * DK + x8 / DV));
          a[gr][jj] = pr.x, su[gr][jj] = pr.y;
        }
      }
#pragma unroll
      for (int gr = 0; gr < NGR; ++gr) {
#pragma unroll
        for (int jj = 0; jj < LB; ++jj) {
          if (j + jj < nagg) {
            const float wf = w[gr] * su[gr][jj];
#pragma unroll
            for (int c = 0; c < 8; ++c) xs[gr][c] += wf * (float)u[gr][jj][c];
            w[gr] *= a[gr][jj];
          }
          consume(u[gr][jj], a[gr][jj]);
          consume(u[gr][jj], su[gr][jj]);
        }
      }
    }
#pragma unroll
    for (int gr = 0; gr < NGR; ++gr) {
      const int x8 = (8 * (tid + kThreads * gr)) % DKDV;
      if (!base_s0) {
        const int r = run - 1 - nagg;
        const half8 u = ld_coh(rI, r * DKDV + x8);
        const float su = ld_dev2(IncP + 2 * (((long)ch * NS + r) * DK + x8 / DV)).y;
        const float wf = w[gr] * su;
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[gr][c] += wf * (float)u[c];
      } else if (s0) {
        float z[8];
        load_f8(s0 + bh * DKDV + x8, z);
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[gr][c] += w[gr] * z[c];
      }
    }
  } else {
#pragma unroll
    for (int gr = 0; gr < NGR; ++gr) {
      const int x8 = (8 * (tid + kThreads * gr)) % DKDV;
      if (s0) {
        load_f8(s0 + bh * DKDV + x8, xs[gr]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[gr][c] = 0.f;
      }
    }
  }

  // -- publish the inclusive state A_run S_in + X (for the next runs, or as
  // the final state), then count this run as done reading
  const bool last = run == NS - 1;
#pragma unroll
  for (int gr = 0; gr < NGR; ++gr) {
    const int x8 = 8 * (tid + kThreads * gr), d = x8 / DV;
    if (x8 < DKDV) {
      const half8 ag = *reinterpret_cast<const half8*>(&sXs[d][x8 % DV]);
      float inc[8], m = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        inc[c] = sAn[d] * xs[gr][c] + sSig[d] * (float)ag[c];
        m = fmaxf(m, fabsf(inc[c]));
      }
      if (last) {
        if (sfin) store_f8(sfin + bh * DKDV + x8, inc);
      } else {
        const float sg = row_scale(DV == 64 ? group_max<8>(m) : group_max<4>(m));
        const float inv = inv_scale(sg);
#pragma unroll
        for (int c = 0; c < 8; ++c) inc[c] *= inv;
        st_coh(rI, run * DKDV + x8, cvt8(inc));
        if (x8 % DV == 0) st_dev2(IncP + 2 * (((long)ch * NS + run) * DK + d), sAn[d], sg);
      }
    }
  }
  if (!last) {
    if (tid == 0) sPub = 0u;
    __syncthreads();
    publish_status(cw + run, kStInc, &sPub);
  }
  if (tid == 0) sDone = atomicAdd(cw + NS, 1u);
  __syncthreads();  // the aggregate in sXs is no longer read; sDone visible
  if (sDone == (unsigned)(NS - 1)) {  // the chain's last run to finish reading
    for (int i = tid; i < NS + 1; i += kThreads) cw[i] = 0u;
  }

  // ===== pass B: S_in into the accumulator layout (through LDS in float),
  // then every chunk in full with S carried along the run
#pragma unroll
  for (int gr = 0; gr < NGR; ++gr) {
    const int x8 = 8 * (tid + kThreads * gr);
    if (x8 < DKDV) store_f8(&sS32[x8 / DV][x8 % DV], xs[gr]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + 4 * i;
    if (blk < NBLK)
      X[i] = *reinterpret_cast<const floatx4*>(&sS32[drow][16 * (blk / ND) + 4 * lq]);
  }
  __syncthreads();  // sS32 read; its region becomes K^ and S again

#pragma nounroll
  for (int g = 0; g < ng; ++g) {
    const int tok0 = (run * G + g) * C;
    if (!kPrefetch) issue(run * G + g, true);
    float qf[NEL], kf[NEL], sc[NEL];
    const bool pad = rpad;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      rq[ks].get(&qf[8 * ks]);
      rk[ks].get(&kf[8 * ks]);
      rg[ks].get(&sc[8 * ks]);
    }
    put_v();
    if (kPrefetch && g + 1 < ng) issue(run * G + g + 1, true);
    if (tid < DK) sRowMax[tid] = 0u;
    if (tok0 + C > T) {
      zero_row<NEL>(pad, qf);
      zero_row<NEL>(pad, kf);
      zero_row<NEL>(pad, sc);
    }
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
    __syncthreads();
    row_max_into_lds(X);  // rows of the state entering this chunk
    // -- per (sub-block, key dim) factors, one key dim per thread
    if (tid < NB * DK) {
      const int I2 = tid / DK, d = tid % DK;
      float tots[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J) tots[J] = sTot[J][d];
      const float s7 = sS7[I2][d];
      float beta = 0.f, tot = 0.f, after = 0.f;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J < I2) beta += tots[J];
        else if (J == I2) tot = tots[J];
        else after += tots[J];
      }
      sEb[I2][d] = fexp2(beta);
      sR1[I2][d] = fexp2(-s7);
      sR2[I2][d] = fexp2(s7 - tot);
      sF[I2][d] = fexp2(after);
      float acc = 0.f;
#pragma unroll
      for (int J = NB - 2; J >= 0; --J) {
        if (J < I2) {
          sM[I2 * (I2 - 1) / 2 + J][d] = fexp2(acc);
          acc += tots[J];
        }
      }
      if (I2 == NB - 1) sAn[d] = fexp2(beta + tot);
    }
    __syncthreads();
    // -- S_n into LDS (rows divided by their scales) for the readout
    stage_rows(X);
    if (tid < DK) sSig[tid] = row_scale(__uint_as_float(sRowMax[tid]));
    // -- per-element factors; K~ and K^ to LDS
    float qt[NEL], kt[NEL];
    float rng = 0.f, big = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float tt[8], ff[8], x1[8], x2[8];
      lds8(&sTot[I][32 * ks + lk], tt);
      lds8(&sF[I][32 * ks + lk], ff);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = 8 * ks + c;
        rng = fmaxf(rng, -tt[c]);
        big = fmaxf(big, fmaxf(fabsf(qf[e]), fabsf(kf[e])));
        qt[e] = qf[e] * fexp2(sc[e]);
        kt[e] = kf[e] * fexp2(tt[c] - sc[e]);
        x1[c] = kt[e];
        x2[c] = kt[e] * ff[c];
      }
      *reinterpret_cast<half8*>(&sKt[t][32 * ks + lk]) = cvt8(x1);
      *reinterpret_cast<half8*>(&sKh[t][32 * ks + lk]) = cvt8(x2);
    }
    __syncthreads();  // K~, K^, S_n and its row scales in LDS

    // -- score sub-blocks: diagonal by this wave's tier, off-diagonal on
    // factors <= 1, scaled down by sigA if needed
    half4 A[NB];
    float sigA = 1.f;
    {
      const float amp = big * fexp2(fminf(rng, 127.f));
      const int tier = __all(rng <= kHalfRange && amp <= 32768.f)  ? 0
                       : __all(rng <= kF32Range && amp < 0x1p126f) ? 1
                                                                    : 2;
      floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
      if (tier == 0) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float r1[8], r2[8], xa[8], xb[8];
          lds8(&sR1[I][32 * ks + lk], r1);
          lds8(&sR2[I][32 * ks + lk], r2);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            xa[c] = qt[8 * ks + c] * r1[c];
            xb[c] = kt[8 * ks + c] * r2[c];
          }
          dacc = mfma16x16x32(cvt8(xb), cvt8(xa), dacc);
        }
      } else if (tier == 1) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float r1[8], r2[8];
          lds8(&sR1[I][32 * ks + lk], r1);
          lds8(&sR2[I][32 * ks + lk], r2);
#pragma unroll
          for (int c = 0; c < 8; ++c)
            dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[8 * ks + c] * r2[c],
                                                        qt[8 * ks + c] * r1[c], dacc, 0, 0, 0);
        }
      } else {
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
      floatx4 Af[NB];
#pragma unroll
      for (int r = 0; r < 4; ++r) dacc[r] = (4 * lq + r <= lr) ? dacc[r] : 0.f;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J == I) Af[J] = dacc;
        else if (J > I) Af[J] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
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
      float am = 0.f;
#pragma unroll
      for (int J = 0; J < NB; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(Af[J][r]));
      if (__any(am > kRowRange)) {
        sigA = row_scale(group_max<64>(am));
        const float inv = inv_scale(sigA);
#pragma unroll
        for (int J = 0; J < NB; ++J) Af[J] *= inv;
      }
#pragma unroll
      for (int J = 0; J < NB; ++J) A[J] = cvt4(Af[J]);
    }
    // -- Q^ = q 2^(b_i), with S_n's row scales folded in when a row is scaled
    const float smax = group_max<64>(sSig[lane % DK]);
    half8 qh[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float eb[8], x[8];
      lds8(&sEb[I][32 * ks + lk], eb);
      if (smax != 1.f) {
        float f[8];
        lds8(&sSig[32 * ks + lk], f);
        const float is = inv_scale(smax);
#pragma unroll
        for (int c = 0; c < 8; ++c) eb[c] *= f[c] * is;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = qt[8 * ks + c] * eb[c];
      qh[ks] = cvt8(x);
    }
    // -- the state after this chunk: S <- diag(a_n) S + K^T V
    {
      const float an = sAn[drow];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int blk = wave + 4 * i;
        if (blk < NBLK) {
          const int E = blk / ND, D = blk % ND;
          X[i] *= an;
#pragma unroll
          for (int J = 0; J < NB; ++J) {
            const half4 a = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            const half4 bb = ld_tr<HSTR, 4>(&sKh[16 * J][16 * D]);
            X[i] = mfma16x16x16(a, bb, X[i]);
          }
        }
      }
    }
    __syncthreads();  // K~ is no longer read: its LDS becomes the output tile
    // -- O = A V + Q^ S_n
    {
      const bool rescale = sigA != 1.f || smax != 1.f;
      const float f1 = sigA * inv_scale(smax);
#pragma unroll
      for (int E = 0; E < NE; ++E) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I) {
            const half4 vb = ld_tr<VSTR, 4>(&sV[16 * J][16 * E]);
            acc = mfma16x16x16(A[J], vb, acc);
          }
        }
        if (rescale) acc *= f1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const half4 sb = ld_tr<SSTR, 8>(&sXs[32 * ks + 4 * hh][16 * E]);
            const half4 qa = hh ? __builtin_shufflevector(qh[ks], qh[ks], 4, 5, 6, 7)
                                : __builtin_shufflevector(qh[ks], qh[ks], 0, 1, 2, 3);
            acc = mfma16x16x16(qa, sb, acc);
          }
        }
        if (smax != 1.f) acc *= smax;
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[16 * I + 4 * lq + r][16 * E + lr] = (InT)acc[r];
      }
    }
    __syncthreads();
    // -- scatter the chunk's rows to their raster positions
    constexpr int LPR = DV / 8;
    for (int u = tid; u < C * LPR; u += kThreads) {
      const int r = u / LPR, c8 = (u % LPR) * 8;
      const int rr = token_row(tok0 + r, T, gh, gw, dir);
      if (rr >= 0) copy8(op + (((long)b * T + rr) * H + h) * DV + c8, &sO[r][c8]);
    }
    __syncthreads();  // every LDS tile of this chunk is free
  }
}

template <int DK, int DV, int C, typename InT, int G>
hipError_t runs_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                  const void* k, const void* v, const void* gk, void* o, char* ws,
                  const float* s0, float* sfin, hipStream_t s) {
  const WsLayout w = workspace_layout(p);
  const int NS = (p.N + G - 1) / G;
  const long nch = (long)nb * p.H;
  const long tok = (long)b0 * p.T * p.H;
  const long bhn = (long)b0 * p.H * p.N;
  const long st = (long)b0 * p.H * DK * DV;
  hipLaunchKernelGGL((runs_kernel<DK, DV, C, InT, G>), dim3((unsigned)(NS * nch)), dim3(kThreads),
                     0, s, static_cast<const InT*>(q) + tok * DK,
                     static_cast<const InT*>(k) + tok * DK, static_cast<const InT*>(v) + tok * DV,
                     static_cast<const InT*>(gk) + tok * DK, static_cast<InT*>(o) + tok * DV,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhn * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_a) + 2 * bhn * DK,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhn * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_g) + 2 * bhn * DK,
                     reinterpret_cast<unsigned*>(ws), s0 ? s0 + st : nullptr,
                     sfin ? sfin + st : nullptr, p.T, p.H, p.N, NS, (int)nch, p.gh, p.gw, dirs);
  return hipGetLastError();
}

}  // namespace tile

bool runs_fit(const Problem& p, int nb) {
  if (p.chunk != 64) return false;
  const long NS = (p.N + kRunChunks - 1) / kRunChunks;
  const long words = kCtrlHeader + (long)nb * p.H * (NS + 1);
  return words <= kCtrlWords && NS * (long)nb * p.H <= 0x7fffffffL;
}

hipError_t launch_runs(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                       const void* k, const void* v, const void* gk, void* o, char* ws,
                       const float* s0, float* sfin, hipStream_t s) {
  using namespace tile;
  constexpr int G = kRunChunks;
  const bool f16 = p.dtype == 0;
  const int key = (p.dk == 64) * 10 + (p.dv == 64);
  if (p.chunk != 64) return hipErrorInvalidValue;
  switch (key) {
    case 0: return f16 ? runs_t<32, 32, 64, half_t, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                       : runs_t<32, 32, 64, float, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 1: return f16 ? runs_t<32, 64, 64, half_t, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                       : runs_t<32, 64, 64, float, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 10: return f16 ? runs_t<64, 32, 64, half_t, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                        : runs_t<64, 32, 64, float, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 11: return f16 ? runs_t<64, 64, 64, half_t, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                        : runs_t<64, 64, 64, float, G>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gla
