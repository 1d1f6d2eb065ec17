// Host-side launch interface between the C-ABI layer (gla_api.hip) and the
// kernels (gla_kernels.hip). Arguments are already validated here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gla_device.h"

namespace gla {

struct Problem {
  int B, H, gh, gw, T, dk, dv, chunk, N;
  int dtype;  // GLA_F16 or GLA_F32
};

// Byte offsets of the intermediate arrays inside the workspace.
struct WsLayout {
  size_t off_U, off_a, off_S, total;
};

WsLayout workspace_layout(const Problem& p);

// Each launcher enqueues one phase for batch elements [b0, b0 + nb) of the
// problem (nb <= kMaxBatchPerLaunch); pointers are the full-problem bases.
hipError_t launch_summaries(const Problem& p, int b0, int nb, const DirPack& dirs,
                            const void* k, const void* v, const void* gk, char* ws,
                            hipStream_t s);
// s0 / sfin (nullable) are the full-problem [B][H][dk][dv] fp32 state arrays.
hipError_t launch_scan(const Problem& p, int b0, int nb, char* ws, const float* s0,
                       float* sfin, hipStream_t s);
hipError_t launch_outputs(const Problem& p, int b0, int nb, const DirPack& dirs,
                          const void* q, const void* k, const void* v, const void* gk,
                          void* o, const char* ws, hipStream_t s);
hipError_t launch_scan_perm(int32_t* perm, int gh, int gw, int dir, hipStream_t s);

}  // namespace gla
