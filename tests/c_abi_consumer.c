/*
 * A plain C program that uses libditnorm.so through include/ditnorm.h only:
 * device memory from the HIP runtime's C API, the library's entry points with
 * raw pointers, no Python, no torch.  tests/test_gpu_c_abi.py writes the
 * inputs, runs this program and compares what it writes with the oracle.
 *
 *   c_abi_consumer DIR
 *
 * DIR/meta.txt holds "rows cols" for a single batch (cols a multiple of 384);
 * DIR/x.bin, scale.bin, shift.bin, d_out.bin, gate.bin and weight.bin hold
 * bf16 bit patterns (rows x cols, cols, cols, rows x cols, cols, cols), and
 * bias.bin and gamma.bin 96 fp32 values.  The program runs
 *   ln_modulate(x, scale, shift)                       -> out.bin
 *   ln_modulate_backward(x, scale, d_out)  (workspace sized by
 *       ln_modulate_backward_workspace_bytes)           -> d_x, d_scale, d_shift.bin
 *   gated_ln_modulate(x, residual = d_out, gate, scale, shift) -> h.bin, gated.bin
 *   rms_modulate(x, weight, scale, shift)              -> rms.bin
 *   qk_layernorm(q = x, k = d_out as rows of 128)      -> q_out.bin, k_out.bin
 *   rmsnorm_silu_bias(x as pixels of 96 channels, bias, gamma) -> wan.bin
 * and checks that a call with a null input fails with
 * DITNORM_INVALID_ARGUMENT and the matching status string.  It exits 0, or
 * prints the failing step and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ditnorm.h"

static char g_dir[4096];

static void *read_file(const char *name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char *name, const void *p, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

#define CHECK_HIP(call)                                                        \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
      return 1;                                                                \
    }                                                                          \
  } while (0)

#define CHECK_DN(call)                                                         \
  do {                                                                         \
    int s_ = (call);                                                           \
    if (s_ != DITNORM_OK) {                                                    \
      fprintf(stderr, "%s returned %d (%s)\n", #call, s_,                      \
              ditnorm_status_string(s_));                                      \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 2 || strlen(argv[1]) >= sizeof g_dir) {
    fprintf(stderr, "usage: c_abi_consumer DIR\n");
    return 1;
  }
  strcpy(g_dir, argv[1]);
  char meta[4200];
  snprintf(meta, sizeof meta, "%s/meta.txt", g_dir);
  FILE *mf = fopen(meta, "r");
  long long rows = 0, cols = 0;
  if (!mf || fscanf(mf, "%lld %lld", &rows, &cols) != 2 || rows <= 0 || cols <= 0) {
    fprintf(stderr, "bad %s\n", meta);
    if (mf) fclose(mf);
    return 1;
  }
  fclose(mf);
  const size_t act = (size_t)rows * (size_t)cols * 2, vec = (size_t)cols * 2;
  uint16_t *x = read_file("x.bin", act), *sc = read_file("scale.bin", vec);
  uint16_t *sh = read_file("shift.bin", vec), *dout = read_file("d_out.bin", act);
  uint16_t *gt = read_file("gate.bin", vec), *wt = read_file("weight.bin", vec);
  float *bias = read_file("bias.bin", 96 * 4), *gamma = read_file("gamma.bin", 96 * 4);
  if (!x || !sc || !sh || !dout || !gt || !wt || !bias || !gamma || cols % 384 != 0) {
    fprintf(stderr, "missing input files in %s, or cols not a multiple of 384\n", g_dir);
    return 1;
  }

  void *dx_in, *dsc, *dsh, *dd, *dout_ln, *ddx, *dws = NULL;
  float *dds, *ddh;
  CHECK_HIP(hipMalloc(&dx_in, act));
  CHECK_HIP(hipMalloc(&dsc, vec));
  CHECK_HIP(hipMalloc(&dsh, vec));
  CHECK_HIP(hipMalloc(&dd, act));
  CHECK_HIP(hipMalloc(&dout_ln, act));
  CHECK_HIP(hipMalloc(&ddx, act));
  CHECK_HIP(hipMalloc((void **)&dds, (size_t)cols * 4));
  CHECK_HIP(hipMalloc((void **)&ddh, (size_t)cols * 4));
  CHECK_HIP(hipMemcpy(dx_in, x, act, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dsc, sc, vec, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dsh, sh, vec, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dd, dout, act, hipMemcpyHostToDevice));

  /* forward: one batch, the modulation rows dense (stride = cols), eps 1e-6,
     no debug outputs, the default stream */
  CHECK_DN(ln_modulate(dx_in, dsc, dsh, dout_ln, rows, cols, rows, cols, 1e-6f, NULL, NULL,
                       NULL, NULL));

  /* backward: the caller's workspace */
  const int64_t ws = ln_modulate_backward_workspace_bytes(rows, cols, rows, DITNORM_DTYPE_BF16);
  if (ws < 0) {
    fprintf(stderr, "ln_modulate_backward_workspace_bytes returned %lld\n", (long long)ws);
    return 1;
  }
  if (ws > 0) CHECK_HIP(hipMalloc(&dws, (size_t)ws));
  CHECK_DN(ln_modulate_backward(dx_in, dsc, dd, ddx, dds, ddh, rows, cols, rows, cols, 1e-6f,
                                dws, ws, NULL, NULL, DITNORM_DTYPE_BF16, NULL));

  /* the other entry points on the same buffers */
  void *dgt, *dwt, *dh, *dgo, *drms, *dqo, *dko, *dwan;
  float *dbias, *dgamma;
  CHECK_HIP(hipMalloc(&dgt, vec));
  CHECK_HIP(hipMalloc(&dwt, vec));
  CHECK_HIP(hipMalloc((void **)&dbias, 96 * 4));
  CHECK_HIP(hipMalloc((void **)&dgamma, 96 * 4));
  CHECK_HIP(hipMalloc(&dh, act));
  CHECK_HIP(hipMalloc(&dgo, act));
  CHECK_HIP(hipMalloc(&drms, act));
  CHECK_HIP(hipMalloc(&dqo, act));
  CHECK_HIP(hipMalloc(&dko, act));
  CHECK_HIP(hipMalloc(&dwan, act));
  CHECK_HIP(hipMemcpy(dgt, gt, vec, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dwt, wt, vec, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dbias, bias, 96 * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dgamma, gamma, 96 * 4, hipMemcpyHostToDevice));
  CHECK_DN(gated_ln_modulate(dx_in, dd, dgt, dsc, dsh, dh, dgo, rows, cols, rows, cols, 1e-6f,
                             NULL, NULL, NULL, NULL));
  CHECK_DN(rms_modulate(dx_in, dwt, dsc, dsh, drms, NULL, NULL, NULL, rows, cols, rows, cols,
                        1e-6f, NULL, NULL, NULL));
  const int64_t heads = rows * cols / 128, pixels = rows * cols / 96;
  CHECK_DN(qk_layernorm(dx_in, dd, dqo, dko, heads, heads, 128, 1e-5f, NULL, NULL, NULL));
  CHECK_DN(rmsnorm_silu_bias(dx_in, dbias, dgamma, dwan, pixels, 96, 1e-6f, NULL, NULL, NULL));

  /* a rejected call: a null input, no launch */
  const int bad = ln_modulate(NULL, dsc, dsh, dout_ln, rows, cols, rows, cols, 1e-6f, NULL,
                              NULL, NULL, NULL);
  if (bad != DITNORM_INVALID_ARGUMENT || strlen(ditnorm_status_string(bad)) == 0) {
    fprintf(stderr, "a null input gave status %d\n", bad);
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());

  uint16_t *out = malloc(act), *dx = malloc(act);
  float *dscale = malloc((size_t)cols * 4), *dshift = malloc((size_t)cols * 4);
  if (!out || !dx || !dscale || !dshift) return 1;
  CHECK_HIP(hipMemcpy(out, dout_ln, act, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dx, ddx, act, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dscale, dds, (size_t)cols * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dshift, ddh, (size_t)cols * 4, hipMemcpyDeviceToHost));
  if (write_file("out.bin", out, act) || write_file("d_x.bin", dx, act) ||
      write_file("d_scale.bin", dscale, (size_t)cols * 4) ||
      write_file("d_shift.bin", dshift, (size_t)cols * 4)) {
    fprintf(stderr, "cannot write outputs to %s\n", g_dir);
    return 1;
  }
  const struct {
    const char *name;
    void *dev;
  } more[] = {{"h.bin", dh},         {"gated.bin", dgo}, {"rms.bin", drms},
              {"q_out.bin", dqo},    {"k_out.bin", dko}, {"wan.bin", dwan}};
  for (size_t i = 0; i < sizeof more / sizeof more[0]; ++i) {
    CHECK_HIP(hipMemcpy(out, more[i].dev, act, hipMemcpyDeviceToHost));
    if (write_file(more[i].name, out, act)) {
      fprintf(stderr, "cannot write %s to %s\n", more[i].name, g_dir);
      return 1;
    }
  }
  printf("c_abi_consumer: %lld x %lld, workspace %lld bytes: ok\n", rows, cols, (long long)ws);
  return 0;
}
