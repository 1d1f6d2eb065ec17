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
  int dtype;   // GLA_F16 or GLA_F32
  int vs = 1;  // single pass: workgroups per chunk-head, each on dv / vs value columns
};

// Byte offsets of the arrays inside the workspace: the control words (fixed
// size, offset 0), U (half rows divided by their scales), the pairs
// (a_n[d], row scale of U_n row d) as float2 [B][H][N][dk] (twice that for
// dv = 64, whose single pass may split the value columns in two), S (S also
// holds the single-pass segment aggregates), the single-pass segment pairs
// (decay, row scale), and the row scales of the three-phase S (float
// [B][H][N][dk]). Every scale is a power of two.
struct WsLayout {
  size_t off_U, off_a, off_S, off_g, off_ss, total;
};

WsLayout workspace_layout(const Problem& p);

// Segments of the single-pass schedule: G chunks each (one segment of N
// chunks up to N = 8, else G = ceil(sqrt(N))).
struct Segments {
  int G, nseg;
};
Segments onepass_segments(int N);
// Whether a launch of nb batch elements fits the single-pass schedule's
// control words and wait width (with p.vs chains per (batch, head)).
bool onepass_fits(const Problem& p, int nb);

// Each launcher enqueues one phase for batch elements [b0, b0 + nb) of the
// problem (nb <= kMaxBatchPerLaunch); pointers are the full-problem bases.
hipError_t launch_summaries(const Problem& p, int b0, int nb, const DirPack& dirs,
                            const void* k, const void* v, const void* gk, char* ws,
                            hipStream_t s);
// s0 / sfin (nullable) are the full-problem [B][H][dk][dv] fp32 state arrays.
hipError_t launch_scan(const Problem& p, int b0, int nb, char* ws, const float* s0,
                       float* sfin, hipStream_t s);
// Optional fused epilogue of the chunk kernels: with gate != nullptr the
// output rows become o / sqrt(mean(o^2) + eps) * weight * silu(gate) (gate
// [B][T][H][dv] in the input dtype, weight float [dv]).
struct Epilogue {
  const void* gate = nullptr;
  const float* weight = nullptr;
  float eps = 0.f;
};

hipError_t launch_outputs(const Problem& p, int b0, int nb, const DirPack& dirs,
                          const void* q, const void* k, const void* v, const void* gk,
                          void* o, const char* ws, const Epilogue& epi, hipStream_t s);
hipError_t launch_outputs_gated(const Problem& p, int b0, int nb, const DirPack& dirs,
                                const void* q, const void* k, const void* v, const void* gk,
                                void* o, const char* ws, const Epilogue& epi, hipStream_t s);
// The whole forward in one kernel (requires onepass_fits(p, nb)).
hipError_t launch_onepass(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                          const void* k, const void* v, const void* gk, void* o, char* ws,
                          const float* s0, float* sfin, const Epilogue& epi, hipStream_t s);
hipError_t launch_onepass_gated(const Problem& p, int b0, int nb, const DirPack& dirs,
                                const void* q, const void* k, const void* v, const void* gk,
                                void* o, char* ws, const float* s0, float* sfin,
                                const Epilogue& epi, hipStream_t s);
// The forward over runs of run_chunks(dtype) chunks per workgroup (one group
// of four waves per chunk) with a decoupled look-back between runs
// (gla_runs.hip). Chunk 64 only; requires runs_fit(p, nb).
int run_chunks(int dtype);
bool runs_fit(const Problem& p, int nb);
hipError_t launch_runs(const Problem& p, int b0, int nb, const DirPack& dirs, const void* q,
                       const void* k, const void* v, const void* gk, void* o, char* ws,
                       const float* s0, float* sfin, hipStream_t s);
// Zero the control words of a workspace (a fill kernel, graph-capturable).
hipError_t launch_ctrl_clear(char* ws, hipStream_t s);
// Spatial SwiGLU core (ssw_kernels.hip): h = silu(a) * (3x3 depthwise conv of u + bias).
hipError_t launch_spatial_swiglu(int dtype, const void* a, const void* u, const float* w,
                                 const float* bias, void* h, int B, int gh, int gw, int F,
                                 hipStream_t s);
hipError_t launch_scan_perm(int32_t* perm, int gh, int gw, int dir, hipStream_t s);

}  // namespace gla
