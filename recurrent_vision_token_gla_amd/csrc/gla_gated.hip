// Instantiations of the chunk kernels with the fused output gate of the GLA
// block (ai.info summary of GTR, "Methodology in Plain English": a
// data-dependent output gate on the RMS-normalised output), compiled apart
// from the plain ones.
#include "gla_chunk.h"

namespace gla {
namespace tile {

template <int DK, int DV, int C, typename InT>
hipError_t outputs_gated(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                         const void* k, const void* v, const void* gk, void* o, const char* ws,
                         const Epilogue& epi, hipStream_t s) {
  return outputs_t<DK, DV, C, InT, true>(p, b0, nb, dirs, q, k, v, gk, o, ws, epi, s);
}

template <int DK, int DV, int C, typename InT>
hipError_t onepass_gated(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                         const void* k, const void* v, const void* gk, void* o, char* ws,
                         const float* s0, float* sfin, const Epilogue& epi, hipStream_t s) {
  return onepass_t<DK, DV, C, InT, true>(p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, epi, s);
}

}  // namespace tile

using namespace tile;

hipError_t launch_outputs_gated(const Problem& p, int b0, int nb, const DirPack& dirs,
                                const void* q, const void* k, const void* v, const void* gk,
                                void* o, const char* ws, const Epilogue& epi, hipStream_t s) {
  GLA_DISPATCH(outputs_gated, p, b0, nb, dirs, q, k, v, gk, o, ws, epi, s);
}

hipError_t launch_onepass_gated(const Problem& p, int b0, int nb, const DirPack& dirs,
                                const void* q, const void* k, const void* v, const void* gk,
                                void* o, char* ws, const float* s0, float* sfin,
                                const Epilogue& epi, hipStream_t s) {
  GLA_DISPATCH(onepass_gated, p, b0, nb, dirs, q, k, v, gk, o, ws, s0, sfin, epi, s);
}

}  // namespace gla
