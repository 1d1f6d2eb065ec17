/*
 * A plain C99 caller of the library (include/gla.h), with no Python and no
 * torch: the boundary as a C program would use it. Test infrastructure.
 *
 *   gla_c_caller host
 *       calls that need no device: version, status strings, workspace sizes
 *       and argument errors returned before any launch; prints "host ok".
 *   gla_c_caller run DIR B H GH GW DK DV CHUNK DIR0 [DIR1 ...]
 *       reads DIR/q.bin, k.bin, v.bin, gk.bin (fp16, [B][T][H][D]), runs
 *       gla_fwd on the device (buffers from hipMalloc, workspace zeroed by
 *       gla_workspace_init, the null stream), writes DIR/o.bin; prints
 *       "run ok" and the schedule gla_fwd took.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gla.h"

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, __VA_ARGS__);       \
      fprintf(stderr, "\n");              \
      return 1;                           \
    }                                     \
  } while (0)

static int host_checks(void) {
  int32_t dir = GLA_L2R;
  void* fake = (void*)(uintptr_t)0x10000;
  CHECK(gla_abi_version() >= 1, "abi version %d", gla_abi_version());
  CHECK(strncmp(gla_status_string(GLA_E_ARG), "GLA_E_ARG", 9) == 0, "status string");
  CHECK(gla_fwd_workspace_bytes(1, 6, 40, 40, 64, 64, 64) >= 65536, "workspace bytes");
  CHECK(gla_fwd_workspace_bytes(1, 6, 40, 40, 48, 64, 64) == 0, "unsupported dk");
  /* a null input is rejected before anything is launched */
  CHECK(gla_fwd(NULL, fake, fake, fake, fake, 1, 1, 4, 4, 32, 32, &dir, 16, GLA_F16, fake,
                (size_t)1 << 30, NULL) == GLA_E_ARG, "null q");
  /* an unknown direction code */
  dir = 7;
  CHECK(gla_fwd(fake, fake, fake, fake, (char*)fake + 4096, 1, 1, 4, 4, 32, 32, &dir, 16, GLA_F16,
                fake, (size_t)1 << 30, NULL) == GLA_E_ARG, "bad direction");
  /* an empty problem is a no-op */
  CHECK(gla_fwd(NULL, NULL, NULL, NULL, NULL, 0, 1, 4, 4, 32, 32, NULL, 16, GLA_F16, NULL, 0,
                NULL) == GLA_OK, "empty batch");
  printf("host ok\n");
  return 0;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int run(int argc, char** argv) {
  CHECK(argc >= 11, "usage: run DIR B H GH GW DK DV CHUNK DIR0 [DIR1 ...]");
  const char* d = argv[2];
  const int B = atoi(argv[3]), H = atoi(argv[4]), gh = atoi(argv[5]), gw = atoi(argv[6]);
  const int dk = atoi(argv[7]), dv = atoi(argv[8]), chunk = atoi(argv[9]);
  CHECK(B > 0 && argc == 10 + B, "need one direction per batch element");
  int32_t* dirs = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  for (int b = 0; b < B; ++b) dirs[b] = atoi(argv[10 + b]);
  const size_t T = (size_t)gh * gw;
  const size_t nk = (size_t)B * T * H * dk * 2, nv = (size_t)B * T * H * dv * 2;
  void* hq = read_file(d, "q.bin", nk);
  void* hk = read_file(d, "k.bin", nk);
  void* hv = read_file(d, "v.bin", nv);
  void* hg = read_file(d, "gk.bin", nk);
  CHECK(hq && hk && hv && hg, "cannot read the inputs under %s", d);
  const size_t wsb = gla_fwd_workspace_bytes(B, H, gh, gw, dk, dv, chunk);
  CHECK(wsb > 0, "unsupported shape");
  void *q, *k, *v, *g, *o, *ws;
  CHECK(hipMalloc(&q, nk) == hipSuccess && hipMalloc(&k, nk) == hipSuccess &&
            hipMalloc(&v, nv) == hipSuccess && hipMalloc(&g, nk) == hipSuccess &&
            hipMalloc(&o, nv) == hipSuccess && hipMalloc(&ws, wsb) == hipSuccess,
        "hipMalloc failed");
  CHECK(hipMemcpy(q, hq, nk, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(k, hk, nk, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(v, hv, nv, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(g, hg, nk, hipMemcpyHostToDevice) == hipSuccess,
        "hipMemcpy to the device failed");
  int st = gla_workspace_init(ws, wsb, NULL);
  CHECK(st == GLA_OK, "gla_workspace_init: %s", gla_status_string(st));
  st = gla_fwd(q, k, v, g, o, B, H, gh, gw, dk, dv, dirs, chunk, GLA_F16, ws, wsb, NULL);
  CHECK(st == GLA_OK, "gla_fwd: %s (%s)", gla_status_string(st), gla_last_error_detail());
  CHECK(hipDeviceSynchronize() == hipSuccess, "hipDeviceSynchronize failed");
  void* ho = malloc(nv);
  CHECK(ho && hipMemcpy(ho, o, nv, hipMemcpyDeviceToHost) == hipSuccess, "hipMemcpy back failed");
  char path[4096];
  snprintf(path, sizeof(path), "%s/o.bin", d);
  FILE* f = fopen(path, "wb");
  CHECK(f && fwrite(ho, 1, nv, f) == nv, "cannot write %s", path);
  fclose(f);
  printf("run ok schedule %d\n", gla_auto_schedule(B, H, gh, gw, dk, dv, chunk));
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(g);
  hipFree(o);
  hipFree(ws);
  free(hq);
  free(hk);
  free(hv);
  free(hg);
  free(ho);
  free(dirs);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 2 && strcmp(argv[1], "run") == 0) return run(argc, argv);
  fprintf(stderr, "usage: gla_c_caller host | run DIR B H GH GW DK DV CHUNK DIR0 [DIR1 ...]\n");
  return 2;
}
