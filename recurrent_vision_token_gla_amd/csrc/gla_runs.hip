// The forward over runs of chunks: one workgroup per run of GR consecutive
// chunks of one (batch, head) chain, one group of four waves per chunk, with
// a decoupled look-back between runs (GTR project page, "A Kernel That Makes
// Recurrence Fast": the chunkwise recurrence carries the state only between
// chunk boundaries; here the quantity carried between workgroups is the
// state entering each run).
//
// Every chunk of the run is processed at once by its own four waves, exactly
// as in the single pass (chunk_kernel with kFused), up to its summary U_n and
// decay a_n, which stay in the workgroup's LDS instead of going to memory:
//   1. the run's last chunk folds the run's summaries into its aggregate
//      (the state after the run when it enters at zero, and the run's decay)
//      and publishes it (status kStAgg); the score blocks follow meanwhile;
//   2. one wave waits for the nearest predecessor run with its inclusive
//      state published and every run in between aggregated (Merrill and
//      Garland's decoupled look-back; lookback_runs), and every chunk folds
//      those tiles into S_in, the state entering the run;
//   3. each chunk forms its own entering state from S_in and the summaries
//      of the run's earlier chunks in LDS, and the run's last chunk publishes
//      the run's inclusive state (status kStInc), or returns the final state;
//   4. each chunk adds the readout and stores its outputs.
// So a chain moves 8 KB aggregates and inclusive states per run instead of
// per chunk, and within a run chunks exchange their states through LDS. A
// run publishes its aggregate without waiting on anything, and workgroups
// are numbered run-major, so the lowest-numbered unfinished workgroup never
// waits on an unfinished one: with in-order dispatch on every XCD the kernel
// cannot deadlock. Every wait is bounded (kSpinLimit polls; running out sets
// the workspace's sticky error bit). Each chain counts its runs once they
// are done reading; the last one clears the chain's words, so they are zero
// between calls.
#include "gla_chunk.h"

namespace gla {
namespace tile {

// chunks per workgroup: as many 64-token chunks as the LDS of one CU holds
template <typename InT>
constexpr int run_chunks() {
  return sizeof(InT) == 2 ? 4 : 3;
}

template <int DK, int DV, int C, typename InT>
hipError_t runs_t(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                  const void* k, const void* v, const void* gk, void* o, char* ws,
                  const float* s0, float* sfin, hipStream_t s) {
  constexpr int GR = run_chunks<InT>();
  const WsLayout w = workspace_layout(p);
  const int NS = (p.N + GR - 1) / GR;  // runs per chain
  const long nch = (long)nb * p.H;
  const long tok = (long)b0 * p.T * p.H;
  const long bhr = (long)b0 * p.H * NS;
  const long st = (long)b0 * p.H * DK * DV;
  // aggregates in the summary region, their (decay, scale) pairs in the pair
  // region; inclusive states in the state region, their pairs in the segment
  // pair region: each region holds a tile (or pair row) per chunk-head, and a
  // chain has fewer runs than chunks
  hipLaunchKernelGGL((chunk_kernel<DK, DV, C, InT, true, false, GR>), dim3((unsigned)(NS * nch)),
                     dim3(kThreads * GR), 0, s, static_cast<const InT*>(q) + tok * DK,
                     static_cast<const InT*>(k) + tok * DK, static_cast<const InT*>(v) + tok * DV,
                     static_cast<const InT*>(gk) + tok * DK, static_cast<InT*>(o) + tok * DV,
                     reinterpret_cast<half_t*>(ws + w.off_U) + bhr * DK * DV,
                     reinterpret_cast<float*>(ws + w.off_a) + 2 * bhr * DK,
                     reinterpret_cast<half_t*>(ws + w.off_S) + bhr * DK * DV, nullptr,
                     reinterpret_cast<float*>(ws + w.off_g) + 2 * bhr * DK,
                     reinterpret_cast<unsigned*>(ws), s0 ? s0 + st : nullptr,
                     sfin ? sfin + st : nullptr, nullptr, nullptr, 0.f, p.T, p.H, p.N, GR, NS,
                     p.gh, p.gw, dirs);
  return hipGetLastError();
}

}  // namespace tile

int run_chunks(int dtype) {
  return dtype == 0 ? tile::run_chunks<half_t>() : tile::run_chunks<float>();
}

bool runs_fit(const Problem& p, int nb) {
  if (p.chunk != 64) return false;
  const long NS = (p.N + run_chunks(p.dtype) - 1) / run_chunks(p.dtype);
  const long words = kCtrlHeader + (long)nb * p.H * (NS + 1);
  return words <= kCtrlWords && NS * (long)nb * p.H <= 0x7fffffffL;
}

hipError_t launch_runs(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                       const void* k, const void* v, const void* gk, void* o, char* ws,
                       const float* s0, float* sfin, hipStream_t s) {
  using namespace tile;
  const bool f16 = p.dtype == 0;
  const int key = (p.dk == 64) * 10 + (p.dv == 64);
  if (p.chunk != 64) return hipErrorInvalidValue;
  switch (key) {
    case 0: return f16 ? runs_t<32, 32, 64, half_t>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                       : runs_t<32, 32, 64, float>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 1: return f16 ? runs_t<32, 64, 64, half_t>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                       : runs_t<32, 64, 64, float>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 10: return f16 ? runs_t<64, 32, 64, half_t>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                        : runs_t<64, 32, 64, float>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
    case 11: return f16 ? runs_t<64, 64, 64, half_t>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s)
                        : runs_t<64, 64, 64, float>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gla
