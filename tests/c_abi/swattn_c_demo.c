/*
 * A plain C99 caller of libswattn.so: no Python, no torch. Used by the tests
 * to show that the C ABI of include/swattn.h is usable on its own.
 *
 *   swattn_c_demo validate
 *       host-side checks only (no device work): bad parameters must come back
 *       as SWATTN_ERR_INVALID_ARG / UNSUPPORTED with a message.
 *   swattn_c_demo run DIR B H n window dilation causal G0 [G1 ...]
 *       reads DIR/{q,k,v}.bin (and DIR/{qg,kg,vg}.bin with global tokens;
 *       bf16 [B,H,n,64] raw), runs one forward through hipMalloc'd buffers
 *       and writes DIR/o.bin (bf16) and DIR/lse.bin (fp32). Window and
 *       dilation are the same for every head; pass G0 = -1 for no globals.
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "swattn.h"

static int expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got, swattn_status_string(got), want);
    return 1;
  }
  if (want != SWATTN_OK && swattn_last_error()[0] == '\0') {
    fprintf(stderr, "%s: no error message\n", what);
    return 1;
  }
  return 0;
}

static int validate(void) {
  int32_t win[2] = {4, 4}, dil[2] = {1, 1}, g[2] = {3, 3};
  swattn_params p;
  swattn_plan* plan = NULL;
  int bad = 0;
  memset(&p, 0, sizeof p);
  p.batch = 1; p.heads = 2; p.n = 16; p.d = 64; p.window = win; p.dilation = dil;
  p.dtype = SWATTN_BF16;
  p.n_global = 2; p.global_idx = g;  /* repeated index */
  bad |= expect(swattn_create(&p, &plan), SWATTN_ERR_INVALID_ARG, "repeated global index");
  p.n_global = 0; p.global_idx = NULL;
  win[1] = 3;                        /* odd window */
  bad |= expect(swattn_create(&p, &plan), SWATTN_ERR_INVALID_ARG, "odd window");
  win[1] = 4;
  p.d = 128;
  bad |= expect(swattn_create(&p, &plan), SWATTN_ERR_UNSUPPORTED, "d = 128");
  p.d = 64;
  p.key_split = 17;
  bad |= expect(swattn_create(&p, &plan), SWATTN_ERR_INVALID_ARG, "key_split 17");
  p.key_split = 0;
  bad |= expect(swattn_create(NULL, &plan), SWATTN_ERR_INVALID_ARG, "NULL params");
  bad |= expect(swattn_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
                SWATTN_ERR_INVALID_ARG, "forward without a plan");
  bad |= expect(swattn_destroy(NULL), SWATTN_OK, "destroy(NULL)");
  if (plan != NULL) { fprintf(stderr, "plan set on failure\n"); bad = 1; }
  if (!bad) printf("validate: ok\n");
  return bad;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); return NULL; }
  void* buf = malloc(bytes);
  if (buf && fread(buf, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); free(buf); buf = NULL; }
  fclose(f);
  return buf;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int bad = fwrite(buf, 1, bytes, f) != bytes;
  fclose(f);
  return bad;
}

#define HIP_OK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "%s failed\n", #x); return 1; } } while (0)

static int run(int argc, char** argv) {
  if (argc < 10) { fprintf(stderr, "run: too few arguments\n"); return 2; }
  const char* dir = argv[2];
  const int B = atoi(argv[3]), H = atoi(argv[4]), n = atoi(argv[5]);
  const int window = atoi(argv[6]), dilation = atoi(argv[7]), causal = atoi(argv[8]);
  int ng = 0;
  int32_t* G = (int32_t*)malloc(sizeof(int32_t) * (size_t)(argc - 9));
  for (int i = 9; i < argc; ++i)
    if (atoi(argv[i]) >= 0) G[ng++] = atoi(argv[i]);
  int32_t* win = (int32_t*)malloc(sizeof(int32_t) * (size_t)H);
  int32_t* dil = (int32_t*)malloc(sizeof(int32_t) * (size_t)H);
  for (int h = 0; h < H; ++h) { win[h] = window; dil[h] = dilation; }

  swattn_params p;
  memset(&p, 0, sizeof p);
  p.batch = B; p.heads = H; p.n = n; p.d = 64; p.window = win; p.dilation = dil;
  p.causal = causal; p.global_idx = ng ? G : NULL; p.n_global = ng; p.dtype = SWATTN_BF16;
  swattn_plan* plan = NULL;
  int st = swattn_create(&p, &plan);
  free(win); free(dil); free(G);  /* the plan keeps its own copies */
  if (st != SWATTN_OK) { fprintf(stderr, "create: %s: %s\n", swattn_status_string(st), swattn_last_error()); return 1; }

  const size_t elems = (size_t)B * H * n * 64, bytes = elems * 2, lbytes = (size_t)B * H * n * 4;
  const char* names[6] = {"q.bin", "k.bin", "v.bin", "qg.bin", "kg.bin", "vg.bin"};
  void* dev[6] = {NULL, NULL, NULL, NULL, NULL, NULL};
  for (int t = 0; t < (ng ? 6 : 3); ++t) {
    void* host = read_file(dir, names[t], bytes);
    if (!host) return 1;
    HIP_OK(hipMalloc(&dev[t], bytes));
    HIP_OK(hipMemcpy(dev[t], host, bytes, hipMemcpyHostToDevice));
    free(host);
  }
  void *o = NULL, *lse = NULL;
  HIP_OK(hipMalloc(&o, bytes));
  HIP_OK(hipMalloc(&lse, lbytes));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  st = swattn_forward(plan, dev[0], dev[1], dev[2], dev[3], dev[4], dev[5], o, (float*)lse, stream);
  if (st != SWATTN_OK) { fprintf(stderr, "forward: %s: %s\n", swattn_status_string(st), swattn_last_error()); return 1; }
  HIP_OK(hipStreamSynchronize(stream));
  void* ho = malloc(bytes);
  void* hl = malloc(lbytes);
  HIP_OK(hipMemcpy(ho, o, bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl, lse, lbytes, hipMemcpyDeviceToHost));
  if (write_file(dir, "o.bin", ho, bytes) || write_file(dir, "lse.bin", hl, lbytes)) return 1;
  free(ho); free(hl);
  for (int t = 0; t < 6; ++t) if (dev[t]) HIP_OK(hipFree(dev[t]));
  HIP_OK(hipFree(o)); HIP_OK(hipFree(lse));
  HIP_OK(hipStreamDestroy(stream));
  if (swattn_destroy(plan) != SWATTN_OK) return 1;
  printf("run: ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "validate") == 0) return validate();
  if (argc >= 2 && strcmp(argv[1], "run") == 0) return run(argc, argv);
  fprintf(stderr, "usage: %s validate | run DIR B H n window dilation causal G0 [G1 ...]\n", argv[0]);
  return 2;
}
