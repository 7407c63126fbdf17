/*
 * moer_route_c: the router's C ABI (include/moer.h) driven from plain C11.
 * There is no C++ here and no Python or torch in the process. Device memory
 * and the stream come from the HIP runtime's C API.
 *
 * It reads one router call's inputs from a file. Then it runs, on one stream:
 *  - moer_route, with the load statistics fused in;
 *  - moer_load_stats on the counts that moer_route wrote;
 *  - moer_bias_update on a device copy of the bias, from the same counts.
 * It writes every output to a second file. With timed_calls > 0 it also
 * times back-to-back moer_route calls, both in device time (events) and in
 * host enqueue time.
 *
 * Input file, little-endian:
 *  - int32 header[12]: magic 0x524F454D, L, T, d, N, K, n_groups,
 *    topk_groups, n_shared, score_fn, dtype, timed_calls;
 *  - float u: the bias step;
 *  - x [L][T][d], then W_g [L][N][d]: bf16 bits or fp32, as dtype says;
 *  - bias [L][N] fp32.
 * Output file, with Kt = K + n_shared and Nb = N + n_shared:
 *  - topk_idx [L][T][Kt] int32, topk_w [L][T][Kt] fp32;
 *  - tok_entropy [L][T] fp32, agg_entropy [L] fp32;
 *  - counts [L][Nb], offsets [L][Nb+1], perm [L][T*Kt], inv_perm [L][T*Kt],
 *    all int32;
 *  - the fused load-statistics records [L], then moer_load_stats' [L]
 *    (moer_load_stats_t, 64 bytes each);
 *  - the bias [L][N] fp32 after moer_bias_update;
 *  - float: device us per timed call; float: host enqueue us per call (both
 *    0 when nothing was timed).
 * Exit status 0 on success. Otherwise it prints the failing call and its
 * status (with moer_last_error()) and returns 1.
 */
#define _POSIX_C_SOURCE 199309L /* clock_gettime */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "moer.h"

#define MAGIC 0x524F454D

#define HIP_OK(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));               \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

#define MOER_OK_(call)                                                                \
  do {                                                                                \
    moer_status s_ = (call);                                                          \
    if (s_ != MOER_OK) {                                                              \
      fprintf(stderr, "%s: %s (%s)\n", #call, moer_status_str(s_), moer_last_error());\
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

/* copies n bytes from the device and appends them to the output file */
static int dump(FILE* f, const void* dev, size_t n) {
  void* h = malloc(n ? n : 1);
  if (h == NULL) return 0;
  int ok = hipMemcpy(h, dev, n, hipMemcpyDeviceToHost) == hipSuccess && write_all(f, h, n);
  free(h);
  return ok;
}

static double now_us(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return ts.tv_sec * 1e6 + ts.tv_nsec * 1e-3;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hd[12];
  float u = 0.f;
  if (!read_all(in, hd, sizeof hd) || !read_all(in, &u, sizeof u) || hd[0] != MAGIC) {
    fprintf(stderr, "bad input header\n");
    fclose(in);
    return 1;
  }
  moer_route_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.n_layers = hd[1];
  desc.T = hd[2];
  desc.d = hd[3];
  desc.N = hd[4];
  desc.K = hd[5];
  desc.n_groups = hd[6];
  desc.topk_groups = hd[7];
  desc.n_shared = hd[8];
  desc.score_fn = hd[9];
  desc.dtype = hd[10];
  desc.input = MOER_IN_HIDDEN;
  desc.bias_mode = MOER_BIAS_SCORE;
  const int timed = hd[11];
  /* the library validates every field; only the host sizes are needed here */
  if (desc.n_layers < 1 || desc.T < 1 || desc.d < 1 || desc.N < 1 || desc.K < 1 ||
      desc.n_shared < 0 || (desc.dtype != MOER_BF16 && desc.dtype != MOER_F32)) {
    fprintf(stderr, "bad shape in the header\n");
    fclose(in);
    return 1;
  }
  const size_t L = (size_t)desc.n_layers, T = (size_t)desc.T, d = (size_t)desc.d;
  const size_t N = (size_t)desc.N, Kt = (size_t)(desc.K + desc.n_shared);
  const size_t Nb = N + (size_t)desc.n_shared;
  const size_t esz = desc.dtype == MOER_BF16 ? 2 : 4;
  const size_t bx = L * T * d * esz, bw = L * N * d * esz, bb = L * N * sizeof(float);

  void* hx = malloc(bx);
  void* hw = malloc(bw);
  void* hb = malloc(bb);
  if (hx == NULL || hw == NULL || hb == NULL || !read_all(in, hx, bx) || !read_all(in, hw, bw) ||
      !read_all(in, hb, bb)) {
    fprintf(stderr, "short input file\n");
    fclose(in);
    return 1;
  }
  fclose(in);

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  void *x, *w, *ws = NULL;
  float *bias, *bias_upd, *topk_w, *tok_h, *agg_h;
  int32_t *topk_idx, *counts, *offsets, *perm, *inv_perm;
  moer_load_stats_t *st_fused, *st_sep;
  HIP_OK(hipMalloc(&x, bx));
  HIP_OK(hipMalloc(&w, bw));
  HIP_OK(hipMalloc((void**)&bias, bb));
  HIP_OK(hipMalloc((void**)&bias_upd, bb));
  HIP_OK(hipMalloc((void**)&topk_idx, L * T * Kt * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&topk_w, L * T * Kt * sizeof(float)));
  HIP_OK(hipMalloc((void**)&tok_h, L * T * sizeof(float)));
  HIP_OK(hipMalloc((void**)&agg_h, L * sizeof(float)));
  HIP_OK(hipMalloc((void**)&counts, L * Nb * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&offsets, L * (Nb + 1) * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&perm, L * T * Kt * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&inv_perm, L * T * Kt * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&st_fused, L * sizeof(moer_load_stats_t)));
  HIP_OK(hipMalloc((void**)&st_sep, L * sizeof(moer_load_stats_t)));
  HIP_OK(hipMemcpy(x, hx, bx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, hw, bw, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(bias, hb, bb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(bias_upd, hb, bb, hipMemcpyHostToDevice));

  const size_t ws_bytes = moer_route_workspace_bytes(&desc);
  if (ws_bytes == 0) {
    fprintf(stderr, "moer_route_workspace_bytes: %s\n", moer_last_error());
    return 1;
  }
  HIP_OK(hipMalloc(&ws, ws_bytes));

  moer_route_io io;
  memset(&io, 0, sizeof io);
  io.x = x;
  io.w_gate = w;
  io.bias = bias;
  io.topk_idx = topk_idx;
  io.topk_w = topk_w;
  io.tok_entropy = tok_h;
  io.agg_entropy = agg_h;
  io.counts = counts;
  io.offsets = offsets;
  io.perm = perm;
  io.inv_perm = inv_perm;
  io.load_stats = st_fused;

  MOER_OK_(moer_route(&desc, &io, ws, ws_bytes, s));
  MOER_OK_(moer_load_stats(counts, desc.n_layers, desc.N, (int32_t)Nb, st_sep, s));
  MOER_OK_(moer_bias_update(bias_upd, counts, desc.n_layers, desc.N, (int32_t)Nb, u, s));
  HIP_OK(hipStreamSynchronize(s));

  float dev_us = 0.f, host_us = 0.f;
  if (timed > 0) {
    /* the same call back to back (no statistics), after a warm-up */
    io.load_stats = NULL;
    for (int i = 0; i < 10; ++i) MOER_OK_(moer_route(&desc, &io, ws, ws_bytes, s));
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipEventRecord(e0, s));
    const double t0 = now_us();
    for (int i = 0; i < timed; ++i) MOER_OK_(moer_route(&desc, &io, ws, ws_bytes, s));
    const double t1 = now_us();
    HIP_OK(hipEventRecord(e1, s));
    HIP_OK(hipEventSynchronize(e1));
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    dev_us = ms * 1e3f / (float)timed;
    host_us = (float)((t1 - t0) / timed);
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
  }

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) {
    fprintf(stderr, "cannot open %s\n", argv[2]);
    return 1;
  }
  int ok = dump(out, topk_idx, L * T * Kt * sizeof(int32_t)) &&
           dump(out, topk_w, L * T * Kt * sizeof(float)) &&
           dump(out, tok_h, L * T * sizeof(float)) && dump(out, agg_h, L * sizeof(float)) &&
           dump(out, counts, L * Nb * sizeof(int32_t)) &&
           dump(out, offsets, L * (Nb + 1) * sizeof(int32_t)) &&
           dump(out, perm, L * T * Kt * sizeof(int32_t)) &&
           dump(out, inv_perm, L * T * Kt * sizeof(int32_t)) &&
           dump(out, st_fused, L * sizeof(moer_load_stats_t)) &&
           dump(out, st_sep, L * sizeof(moer_load_stats_t)) && dump(out, bias_upd, bb) &&
           write_all(out, &dev_us, sizeof dev_us) && write_all(out, &host_us, sizeof host_us);
  if (fclose(out) != 0) ok = 0;
  if (!ok) {
    fprintf(stderr, "writing %s failed\n", argv[2]);
    return 1;
  }
  if (timed > 0) printf("%d calls: %.2f us per call on the device, %.2f us host enqueue\n", timed,
                        dev_us, host_us);

  void* bufs[] = {x,   w,     bias,    bias_upd, topk_idx, topk_w,   tok_h,  agg_h,
                  counts, offsets, perm, inv_perm, st_fused, st_sep, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(s));
  free(hx);
  free(hw);
  free(hb);
  return 0;
}
