// C ABI of the chunkwise key-only GLA forward (declared in include/gla.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues kernels on the caller's stream. Nothing here allocates,
// synchronises or reads device memory, so the calls are graph-capturable.
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "gla.h"
#include "gla_launch.h"

namespace {

thread_local char g_detail[256] = "";

// Workspaces whose control words gla_workspace_init has zeroed (start address
// -> bytes). The single pass trusts those words only on such a workspace; any
// other workspace runs the three phases, which read no control words, so a
// workspace of arbitrary contents always gives correct results.
std::mutex g_prepared_mu;
std::unordered_map<uintptr_t, size_t> g_prepared;

bool is_prepared(const void* ws) {
  std::lock_guard<std::mutex> lk(g_prepared_mu);
  const auto it = g_prepared.find(reinterpret_cast<uintptr_t>(ws));
  return it != g_prepared.end() && it->second >= (size_t)gla::kCtrlWords * sizeof(unsigned);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int fail_hip(hipError_t e, const char* where) {
  snprintf(g_detail, sizeof(g_detail), "%s: %s", where, hipGetErrorString(e));
  return GLA_E_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape check shared by every entry point. Returns GLA_OK and fills `p`, or
// an error status. `empty` is set when there is nothing to compute.
int make_problem(int B, int H, int gh, int gw, int dk, int dv, int chunk, int dtype,
                 gla::Problem* p, bool* empty) {
  if (B < 0 || H < 0 || gh < 0 || gw < 0) return GLA_E_ARG;
  if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_E_ARG;
  if ((dk != 32 && dk != 64) || (dv != 32 && dv != 64)) return GLA_E_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GLA_E_UNSUPPORTED;
  const long long T = (long long)gh * gw;
  // element offsets are formed in 64-bit; T and the grid counts must fit int
  if (T > 0x7fffffffLL || (long long)B * T * H > (1LL << 40)) return GLA_E_UNSUPPORTED;
  *empty = (B == 0 || H == 0 || T == 0);
  p->B = B; p->H = H; p->gh = gh; p->gw = gw; p->T = (int)T;
  p->dk = dk; p->dv = dv; p->chunk = chunk; p->dtype = dtype;
  p->N = (int)((T + chunk - 1) / chunk);
  if (!*empty && (p->N > 0x7fffffff / 1 || H > 65535)) return GLA_E_UNSUPPORTED;
  return GLA_OK;
}

int check_dirs(const int32_t* dir, int B) {
  if (!dir) return GLA_E_ARG;
  for (int b = 0; b < B; ++b)
    if (dir[b] < GLA_L2R || dir[b] > GLA_B2T) return GLA_E_ARG;
  return GLA_OK;
}

gla::DirPack pack_dirs(const int32_t* dir, int b0, int nb) {
  gla::DirPack d;
  memset(&d, 0, sizeof(d));
  for (int i = 0; i < nb; ++i) d.w[i >> 4] |= (uint32_t)(dir[b0 + i] & 3) << (2 * (i & 15));
  return d;
}

int check_ws(const gla::Problem& p, const void* ws, size_t ws_bytes) {
  const gla::WsLayout w = gla::workspace_layout(p);
  if (!ws) return GLA_E_ARG;
  if (!aligned(ws, 256)) return GLA_E_ARG;
  if (ws_bytes < w.total) return GLA_E_WORKSPACE;
  return GLA_OK;
}

int check_tensor(const void* t) { return (t && aligned(t, 16)) ? GLA_OK : GLA_E_ARG; }

#define GLA_TRY(expr)            \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != GLA_OK) return rc_; \
  } while (0)

// Auto dispatch: the single pass saves two kernel boundaries and one read of
// k, v, gk, but every chunk reads O(sqrt(N)) published tiles. Measured on
// MI355X (64/64, chunk 64, graph-replayed over rotating inputs), single pass
// against three phases, in us per call: chains of 25 chunks 13.5 vs 16.2 at
// 150 chunk-heads, 47.7 vs 55.5 at 2,400, 166 vs 188 at 9,600; chains of 49
// chunks 16.9 vs 20.7 at 294, 160 vs 186 at 9,408; chains of 64 chunks 19.3
// vs 21.8 at 384, 116 vs 122 at 6,144; chains of 100 chunks 26.6 vs 25.8 at
// 600, 65.6 vs 58.0 at 2,400, 128 vs 122 at 6,400, 240 vs 243 at 12,800;
// chains of 144 chunks 39.0 vs 34.9 at 864, 183 vs 197 at 9,216; chains of
// 256 chunks 60.8 vs 45.8 at 1,536. Long chains favour the single pass only
// on large grids, about where chunk-heads x N reaches 1.2e6.
constexpr int kOnepassAnyGrid = 64;         // chains this short: single pass at any grid
constexpr int kOnepassMaxChain = 144;       // longest chain measured to gain on large grids
constexpr long kOnepassLongWork = 1200000;  // chunk-heads x N from which those gain

bool single_pass_fits(const gla::Problem& p) {
  const int nb_max = p.B < gla::kMaxBatchPerLaunch ? p.B : gla::kMaxBatchPerLaunch;
  return gla::onepass_fits(p, nb_max);
}

// Value splits of the single pass: every column of the state is its own
// recurrence, so two workgroups per chunk-head can each take half of dv = 64
// (the pages' operator description fixes no work split; the score tile and
// the decay factors are recomputed by both). Worth it only while the grid
// leaves CUs idle: measured on MI355X (64/64, chunk 64, graph-replayed over
// rotating inputs, us per call, unsplit against split), 12.9 vs 11.1 at 54
// chunk-heads, 13.1 vs 11.4 at 96, 12.8 vs 11.1 at 100, 13.0 vs 11.8 at 150,
// 15.5 vs 14.5 at 216 (chains of 36 chunks), 13.4 vs 13.5 at 200, 14.6 vs
// 14.5 at 250, 16.4 vs 17.1 at 294, 14.8 vs 15.7 at 300.
constexpr long kSplitMaxChunks = 224;  // chunk-heads of the whole call

int single_pass_splits(const gla::Problem& p, const gla::Epilogue& epi) {
  if (p.dv != 64 || epi.gate || (long)p.B * p.H * p.N > kSplitMaxChunks) return 1;
  gla::Problem q = p;
  q.vs = 2;
  return single_pass_fits(q) ? 2 : 1;
}

bool prefer_single_pass(const gla::Problem& p) {
  return p.N <= kOnepassAnyGrid ||
         (p.N <= kOnepassMaxChain && (long)p.B * p.H * p.N * p.N >= kOnepassLongWork);
}

int outputs_impl(const void* q, const void* k, const void* v, const void* gk, void* o, int B,
                 int H, int grid_h, int grid_w, int dk, int dv, const int32_t* dir, int chunk,
                 int dtype, void* workspace, size_t workspace_bytes, const gla::Epilogue& epi,
                 void* stream) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, dtype, &p, &empty));
  if (empty) return GLA_OK;
  GLA_TRY(check_tensor(q));
  GLA_TRY(check_tensor(k));
  GLA_TRY(check_tensor(v));
  GLA_TRY(check_tensor(gk));
  GLA_TRY(check_tensor(o));
  if (o == q || o == k || o == v || o == gk) return GLA_E_ARG;
  GLA_TRY(check_dirs(dir, B));
  GLA_TRY(check_ws(p, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < B; b0 += gla::kMaxBatchPerLaunch) {
    const int nb = B - b0 < gla::kMaxBatchPerLaunch ? B - b0 : gla::kMaxBatchPerLaunch;
    const hipError_t e = gla::launch_outputs(p, b0, nb, pack_dirs(dir, b0, nb), q, k, v, gk,
                                             o, static_cast<const char*>(workspace), epi, s);
    if (e != hipSuccess) return fail_hip(e, "chunk outputs launch");
  }
  return GLA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, const void* gk, void* o, int B, int H,
             int grid_h, int grid_w, int dk, int dv, const int32_t* dir, int chunk, int dtype,
             const float* s0, float* s_final, void* workspace, size_t workspace_bytes,
             void* stream, int mode /* 0 auto, 1 single pass, 2 three phases */,
             const gla::Epilogue& epi = gla::Epilogue()) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, dtype, &p, &empty));
  if (empty) return GLA_OK;
  // validate everything before the first launch so that a bad call enqueues nothing
  GLA_TRY(check_tensor(q));
  GLA_TRY(check_tensor(k));
  GLA_TRY(check_tensor(v));
  GLA_TRY(check_tensor(gk));
  GLA_TRY(check_tensor(o));
  if (o == q || o == k || o == v || o == gk) return GLA_E_ARG;
  if (s0) GLA_TRY(check_tensor(s0));
  if (s_final) {
    GLA_TRY(check_tensor(s_final));
    const void* sf = s_final;
    if (sf == q || sf == k || sf == v || sf == gk || sf == o || sf == workspace) return GLA_E_ARG;
  }
  // s_final may be s0 (an in-place update) but must not otherwise overlap it
  const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
  const bool in_place = s0 && s_final && overlaps(s0, state_bytes, s_final, state_bytes);
  if (in_place && (const void*)s0 != (const void*)s_final) return GLA_E_ARG;
  if (epi.gate) {
    GLA_TRY(check_tensor(epi.gate));
    if (!epi.weight || !aligned(epi.weight, 16)) return GLA_E_ARG;
    if (o == epi.gate || !(epi.eps >= 0.f)) return GLA_E_ARG;
  }
  GLA_TRY(check_dirs(dir, B));
  GLA_TRY(check_ws(p, workspace, workspace_bytes));
  // In the single pass the chain's last chunk writes S_T while other chunks
  // of the chain may still read s0, so an in-place update takes the three
  // phases, whose scan reads each element of s0 before it writes the same
  // element of s_final.
  const bool prepared = is_prepared(workspace);
  if (mode == GLA_SCHED_RUNS) {  // runs of chunks with a decoupled look-back
    const int nb_max = B < gla::kMaxBatchPerLaunch ? B : gla::kMaxBatchPerLaunch;
    if (in_place || epi.gate || !gla::runs_fit(p, nb_max)) return GLA_E_UNSUPPORTED;
    if (!prepared) {
      snprintf(g_detail, sizeof(g_detail),
               "the single pass needs a workspace prepared by gla_workspace_init");
      return GLA_E_UNPREPARED;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int b0 = 0; b0 < B; b0 += gla::kMaxBatchPerLaunch) {
      const int nb = B - b0 < gla::kMaxBatchPerLaunch ? B - b0 : gla::kMaxBatchPerLaunch;
      const hipError_t e = gla::launch_runs(p, b0, nb, pack_dirs(dir, b0, nb), q, k, v, gk, o,
                                            static_cast<char*>(workspace), s0, s_final, s);
      if (e != hipSuccess) return fail_hip(e, "runs launch");
    }
    return GLA_OK;
  }
  bool onepass = single_pass_fits(p) && !in_place;
  if (mode == 1 && !onepass) return GLA_E_UNSUPPORTED;
  if (mode == 1 && !prepared) {
    snprintf(g_detail, sizeof(g_detail),
             "the single pass needs a workspace prepared by gla_workspace_init");
    return GLA_E_UNPREPARED;
  }
  onepass = onepass && prepared;
  if (mode == 0) onepass = onepass && prefer_single_pass(p);
  if (mode == 2) onepass = false;
  if (onepass) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    p.vs = single_pass_splits(p, epi);
    for (int b0 = 0; b0 < B; b0 += gla::kMaxBatchPerLaunch) {
      const int nb = B - b0 < gla::kMaxBatchPerLaunch ? B - b0 : gla::kMaxBatchPerLaunch;
      const hipError_t e = gla::launch_onepass(p, b0, nb, pack_dirs(dir, b0, nb), q, k, v, gk, o,
                                               static_cast<char*>(workspace), s0, s_final, epi, s);
      if (e != hipSuccess) return fail_hip(e, "single-pass launch");
    }
    return GLA_OK;
  }
  GLA_TRY(gla_chunk_summaries(k, v, gk, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype,
                              workspace, workspace_bytes, stream));
  GLA_TRY(gla_state_scan(B, H, grid_h, grid_w, dk, dv, chunk, s0, s_final, workspace,
                         workspace_bytes, stream));
  return outputs_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, workspace,
                      workspace_bytes, epi, stream);
}

// ---- allocation-free forward ----------------------------------------------
// gla_fwd_noalloc takes its workspace from this file-scope device array, one
// copy per GPU the library runs on (kept until the process ends). Host code
// never passes the array's name to a kernel: the per-device address from
// hipGetSymbolAddress is kept below and used instead.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The calling thread's current device's copy of `scratch`: on its first use on
// a device, the address is looked up, the control words are zeroed by a kernel
// on `stream` (ordered before the call that needs them) and the address is
// recorded as a prepared workspace. Returns GLA_OK or GLA_E_HIP/_UNSUPPORTED.
int scratch_for_device(hipStream_t stream, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return GLA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    e = gla::launch_ctrl_clear(static_cast<char*>(ptr), stream);
    if (e != hipSuccess) return fail_hip(e, "scratch control-word clear");
    {
      std::lock_guard<std::mutex> lk2(g_prepared_mu);
      g_prepared[reinterpret_cast<uintptr_t>(ptr)] = kScratchBytes;
    }
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return GLA_OK;
}

}  // namespace

extern "C" {

int gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* gk, void* o, int B,
                    int H, int grid_h, int grid_w, int dk, int dv, const int32_t* dir, int chunk,
                    int dtype, void* stream) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, dtype, &p, &empty));
  if (empty) return GLA_OK;
  const size_t need = gla::workspace_layout(p).total;
  if (need > kScratchBytes) {
    snprintf(g_detail, sizeof(g_detail),
             "this problem needs %zu bytes of workspace; the allocation-free forward's "
             "static scratch holds %zu (use gla_fwd with a caller workspace)",
             need, kScratchBytes);
    return GLA_E_WORKSPACE;
  }
  char* ws = nullptr;
  GLA_TRY(scratch_for_device(static_cast<hipStream_t>(stream), &ws));
  return fwd_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, nullptr,
                  nullptr, ws, kScratchBytes, stream, 0);
}

int gla_abi_version(void) { return 5; }

size_t gla_fwd_workspace_bytes(int B, int H, int grid_h, int grid_w, int dk, int dv,
                               int chunk) {
  gla::Problem p;
  bool empty;
  if (make_problem(B, H, grid_h, grid_w, dk, dv, chunk, GLA_F16, &p, &empty) != GLA_OK)
    return 0;
  if (empty) return 0;
  return gla::workspace_layout(p).total;
}

int gla_workspace_layout(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                         size_t* off_U, size_t* off_a, size_t* off_S, size_t* off_scales,
                         size_t* total_bytes) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, GLA_F16, &p, &empty));
  if (!off_U || !off_a || !off_S || !off_scales || !total_bytes) return GLA_E_ARG;
  const gla::WsLayout w = gla::workspace_layout(p);
  *off_U = w.off_U;
  *off_a = w.off_a;
  *off_S = w.off_S;
  *off_scales = w.off_ss;
  *total_bytes = empty ? 0 : w.total;
  return GLA_OK;
}

int gla_chunk_summaries(const void* k, const void* v, const void* gk, int B, int H,
                        int grid_h, int grid_w, int dk, int dv, const int32_t* dir,
                        int chunk, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, dtype, &p, &empty));
  if (empty) return GLA_OK;
  GLA_TRY(check_tensor(k));
  GLA_TRY(check_tensor(v));
  GLA_TRY(check_tensor(gk));
  GLA_TRY(check_dirs(dir, B));
  GLA_TRY(check_ws(p, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < B; b0 += gla::kMaxBatchPerLaunch) {
    const int nb = B - b0 < gla::kMaxBatchPerLaunch ? B - b0 : gla::kMaxBatchPerLaunch;
    const hipError_t e = gla::launch_summaries(p, b0, nb, pack_dirs(dir, b0, nb), k, v, gk,
                                               static_cast<char*>(workspace), s);
    if (e != hipSuccess) return fail_hip(e, "chunk summaries launch");
  }
  return GLA_OK;
}

int gla_state_scan(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                   const float* s0, float* s_final, void* workspace, size_t workspace_bytes,
                   void* stream) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, GLA_F16, &p, &empty));
  if (empty) return GLA_OK;
  if (s0) GLA_TRY(check_tensor(s0));
  if (s_final) GLA_TRY(check_tensor(s_final));
  GLA_TRY(check_ws(p, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < B; b0 += gla::kMaxBatchPerLaunch) {
    const int nb = B - b0 < gla::kMaxBatchPerLaunch ? B - b0 : gla::kMaxBatchPerLaunch;
    const hipError_t e =
        gla::launch_scan(p, b0, nb, static_cast<char*>(workspace), s0, s_final, s);
    if (e != hipSuccess) return fail_hip(e, "boundary scan launch");
  }
  return GLA_OK;
}

int gla_chunk_outputs(const void* q, const void* k, const void* v, const void* gk, void* o,
                      int B, int H, int grid_h, int grid_w, int dk, int dv,
                      const int32_t* dir, int chunk, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return outputs_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, workspace,
                      workspace_bytes, gla::Epilogue(), stream);
}

int gla_fwd(const void* q, const void* k, const void* v, const void* gk, void* o, int B, int H,
            int grid_h, int grid_w, int dk, int dv, const int32_t* dir, int chunk, int dtype,
            void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, nullptr,
                  nullptr, workspace, workspace_bytes, stream, 0);
}

int gla_fwd_state(const void* q, const void* k, const void* v, const void* gk, void* o, int B,
                  int H, int grid_h, int grid_w, int dk, int dv, const int32_t* dir, int chunk,
                  int dtype, const float* s0, float* s_final, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, s0, s_final,
                  workspace, workspace_bytes, stream, 0);
}

int gla_fwd_schedule(const void* q, const void* k, const void* v, const void* gk, void* o, int B,
                     int H, int grid_h, int grid_w, int dk, int dv, const int32_t* dir,
                     int chunk, int dtype, const float* s0, float* s_final, int schedule,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (schedule != GLA_SCHED_AUTO && schedule != GLA_SCHED_SINGLE_PASS &&
      schedule != GLA_SCHED_THREE_PHASE && schedule != GLA_SCHED_RUNS)
    return GLA_E_ARG;
  return fwd_impl(q, k, v, gk, o, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, s0, s_final,
                  workspace, workspace_bytes, stream, schedule);
}

int gla_fwd_gated(const void* q, const void* k, const void* v, const void* gk, const void* gate,
                  const float* norm_weight, float eps, void* y, int B, int H, int grid_h,
                  int grid_w, int dk, int dv, const int32_t* dir, int chunk, int dtype,
                  const float* s0, float* s_final, void* workspace, size_t workspace_bytes,
                  void* stream) {
  gla::Epilogue epi;
  epi.gate = gate;
  epi.weight = norm_weight;
  epi.eps = eps;
  if (!gate) return GLA_E_ARG;
  return fwd_impl(q, k, v, gk, y, B, H, grid_h, grid_w, dk, dv, dir, chunk, dtype, s0, s_final,
                  workspace, workspace_bytes, stream, 0, epi);
}

int gla_auto_schedule(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk) {
  gla::Problem p;
  bool empty;
  GLA_TRY(make_problem(B, H, grid_h, grid_w, dk, dv, chunk, GLA_F16, &p, &empty));
  if (empty) return GLA_SCHED_THREE_PHASE;
  return single_pass_fits(p) && prefer_single_pass(p) ? GLA_SCHED_SINGLE_PASS
                                                       : GLA_SCHED_THREE_PHASE;
}

int gla_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return GLA_E_ARG;
  if (workspace_bytes < (size_t)gla::kCtrlWords * sizeof(unsigned)) return GLA_E_WORKSPACE;
  const hipError_t e =
      gla::launch_ctrl_clear(static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "workspace init launch");
  std::lock_guard<std::mutex> lk(g_prepared_mu);
  g_prepared[reinterpret_cast<uintptr_t>(workspace)] = workspace_bytes;
  return GLA_OK;
}

int gla_workspace_release(const void* workspace) {
  if (!workspace) return GLA_E_ARG;
  std::lock_guard<std::mutex> lk(g_prepared_mu);
  g_prepared.erase(reinterpret_cast<uintptr_t>(workspace));
  return GLA_OK;
}

int gla_workspace_is_prepared(const void* workspace) {
  return workspace && is_prepared(workspace) ? 1 : 0;
}

int gla_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* error_bits, int clear,
                         void* stream) {
  if (!workspace || !aligned(workspace, 256) || !error_bits) return GLA_E_ARG;
  if (workspace_bytes < (size_t)gla::kCtrlWords * sizeof(unsigned)) return GLA_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "workspace status read");
  *error_bits = word;
  if (clear && word != 0u) {
    static const uint32_t zero = 0u;
    e = hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail_hip(e, "workspace status clear");
  }
  return GLA_OK;
}

int gla_scan_perm(int32_t* perm_dev, int grid_h, int grid_w, int dir, void* stream) {
  if (grid_h < 0 || grid_w < 0) return GLA_E_ARG;
  if (dir < GLA_L2R || dir > GLA_B2T) return GLA_E_ARG;
  const long long T = (long long)grid_h * grid_w;
  if (T == 0) return GLA_OK;
  if (T > 0x7fffffffLL) return GLA_E_UNSUPPORTED;
  if (!perm_dev || !aligned(perm_dev, 4)) return GLA_E_ARG;
  const hipError_t e =
      gla::launch_scan_perm(perm_dev, grid_h, grid_w, dir, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "scan perm launch");
  return GLA_OK;
}

int gla_spatial_swiglu(const void* a, const void* u, const float* weight, const float* bias,
                       void* h, int B, int grid_h, int grid_w, int F, int dtype, void* stream) {
  if (B < 0 || grid_h < 0 || grid_w < 0 || F < 0) return GLA_E_ARG;
  if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_E_ARG;
  if (F % 8 != 0) return GLA_E_UNSUPPORTED;
  const long long T = (long long)grid_h * grid_w;
  if (T > 0x7fffffffLL || (long long)B * T * F > (1LL << 40) || B > 65535) return GLA_E_UNSUPPORTED;
  if (B == 0 || T == 0 || F == 0) return GLA_OK;
  GLA_TRY(check_tensor(a));
  GLA_TRY(check_tensor(u));
  GLA_TRY(check_tensor(h));
  if (!weight || !aligned(weight, 4) || (bias && !aligned(bias, 4))) return GLA_E_ARG;
  if (h == a || h == u) return GLA_E_ARG;
  const hipError_t e = gla::launch_spatial_swiglu(dtype, a, u, weight, bias, h, B, grid_h, grid_w,
                                                  F, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "spatial swiglu launch");
  return GLA_OK;
}

const char* gla_status_string(int status) {
  switch (status) {
    case GLA_OK: return "GLA_OK";
    case GLA_E_ARG: return "GLA_E_ARG: invalid argument (null/misaligned pointer, negative size, bad code, aliasing)";
    case GLA_E_UNSUPPORTED: return "GLA_E_UNSUPPORTED: dk, dv or chunk outside the supported set, or problem too large";
    case GLA_E_WORKSPACE: return "GLA_E_WORKSPACE: workspace smaller than gla_fwd_workspace_bytes() (see gla_last_error_detail)";
    case GLA_E_HIP: return "GLA_E_HIP: a HIP launch failed (see gla_last_error_detail)";
    case GLA_E_UNPREPARED: return "GLA_E_UNPREPARED: the single pass needs a workspace prepared by gla_workspace_init";
    default: return "unknown GLA status";
  }
}

const char* gla_last_error_detail(void) { return g_detail; }

}  // extern "C"
