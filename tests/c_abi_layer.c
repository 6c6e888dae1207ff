/*
 * A C99 consumer of the library's C ABI (include/moe.h), with no Python and
 * no torch: it runs the MoE layer's forward pass -- router logits, top-k
 * softmax routing, counting and index generation, GEMM 1 with the SwiGLU
 * epilogue reading x through the row map, GEMM 2, the weighted combine --
 * and its backward pass (the combine's gradient read through the row map,
 * as the Python layer does by default) on device buffers it allocates
 * itself with the HIP runtime, on one stream.
 *
 *   c_abi_layer --check-host   host-only calls (version, validation errors,
 *                              workspace sizes, kernel plans); no GPU needed
 *   c_abi_layer IN OUT         forward and backward pass on the inputs in
 *                              IN, results to OUT (formats below); exit 0
 *                              on success
 *
 * IN  (little-endian): int32 magic 0x31454F4D, T, d, E, k, F; then bf16 bit
 *     patterns (uint16) of x [T, d], wr [d, E], W1 [E, d, 2F], W2 [E, F, d],
 *     dy [T, d].
 * OUT: logits float32 [T, E], topk_idx int32 [T, k], topk_w float32 [T, k],
 *      offsets int32 [E + 1], y bf16 bits [T, d], dx bf16 bits [T, d],
 *      dWr float32 [d, E], dW1 float32 [E, d, 2F], dW2 float32 [E, F, d],
 *      index-error mask uint32 (after the forward, then after the backward).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

#define FAIL(...)                     \
  do {                                \
    fprintf(stderr, __VA_ARGS__);     \
    fputc('\n', stderr);              \
    exit(2);                          \
  } while (0)

#define CHECK_MOE(call)                                                          \
  do {                                                                           \
    moe_status s_ = (call);                                                      \
    if (s_ != MOE_OK) FAIL("%s -> %d: %s", #call, (int)s_, moe_last_error());    \
  } while (0)

#define CHECK_HIP(call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) FAIL("%s -> %s", #call, hipGetErrorString(e_));       \
  } while (0)

static int check_host(void) {
  const char* v = moe_version();
  if (v == NULL || v[0] == '\0') FAIL("empty version string");
  /* Validation happens on the host before anything is enqueued. */
  moe_status s = moe_route_topk(NULL, NULL, 0, 8, 2, 0, NULL, NULL, NULL, NULL, NULL);
  if (s != MOE_ERR_INVALID_ARG) FAIL("moe_route_topk(T=0) returned %d", (int)s);
  if (moe_last_error()[0] == '\0') FAIL("no message after a failed call");
  s = moe_count_index(NULL, 16, 3, 2, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  if (s != MOE_ERR_INVALID_ARG) FAIL("moe_count_index(k > E) returned %d", (int)s);
  s = moe_act_fwd(NULL, 4, 12, MOE_BF16, NULL, NULL);
  if (s == MOE_OK) FAIL("moe_act_fwd accepted F %% 8 != 0");
  if (moe_count_index_workspace_size(8192, 8, 64) == 0) FAIL("zero count/index workspace");
  int tm = 0, tn = 0, wm = 0, wn = 0, split = 0, mfma = -1;
  CHECK_MOE(moe_grouped_gemm_plan(3, 65536, 2048, 2048, 64, MOE_BF16, &tm, &tn, &wm, &wn,
                                  &split, &mfma));
  if (mfma != 1 || tm <= 0 || tn <= 0 || wm * wn <= 0) FAIL("unexpected plan");
  printf("host ok: %s, plan %dx%d tiles, %dx%d waves\n", v, tm, tn, wm, wn);
  return 0;
}

static void* read_exact(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL || fread(p, 1, bytes, f) != bytes) FAIL("short input file");
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (host != NULL) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void from_device(FILE* f, const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (h == NULL) FAIL("out of host memory");
  CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, bytes, f) != bytes) FAIL("short write");
  free(h);
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "--check-host") == 0) return check_host();
  if (argc != 3) FAIL("usage: %s --check-host | IN OUT", argv[0]);

  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) FAIL("cannot open %s", argv[1]);
  int32_t hdr[6];
  if (fread(hdr, sizeof hdr, 1, in) != 1 || hdr[0] != 0x31454F4D) FAIL("bad input header");
  const int T = hdr[1], d = hdr[2], E = hdr[3], k = hdr[4], F = hdr[5];
  const size_t Tk = (size_t)T * (size_t)k;
  const size_t b2 = sizeof(uint16_t);
  void* hx = read_exact(in, (size_t)T * d * b2);
  void* hwr = read_exact(in, (size_t)d * E * b2);
  void* hw1 = read_exact(in, (size_t)E * d * 2 * F * b2);
  void* hw2 = read_exact(in, (size_t)E * F * d * b2);
  void* hdy = read_exact(in, (size_t)T * d * b2);
  fclose(in);

  void* x = to_device(hx, (size_t)T * d * b2);
  void* wr = to_device(hwr, (size_t)d * E * b2);
  void* w1 = to_device(hw1, (size_t)E * d * 2 * F * b2);
  void* w2 = to_device(hw2, (size_t)E * F * d * b2);
  void* dy = to_device(hdy, (size_t)T * d * b2);
  const int32_t router_off_h[2] = {0, T};
  int32_t* router_off = (int32_t*)to_device(router_off_h, sizeof router_off_h);
  float* logits = (float*)to_device(NULL, (size_t)T * E * 4);
  int32_t* idx = (int32_t*)to_device(NULL, Tk * 4);
  float* w = (float*)to_device(NULL, Tk * 4);
  float* probs = (float*)to_device(NULL, (size_t)T * E * 4);
  int32_t* counts = (int32_t*)to_device(NULL, (size_t)E * 4);
  int32_t* offsets = (int32_t*)to_device(NULL, (size_t)(E + 1) * 4);
  int32_t* dest = (int32_t*)to_device(NULL, Tk * 4);
  int32_t* src = (int32_t*)to_device(NULL, Tk * 4);
  const size_t ci_bytes = moe_count_index_workspace_size(T, k, E);
  void* ci_ws = to_device(NULL, ci_bytes);
  void* h = to_device(NULL, Tk * 2 * F * b2);
  void* a = to_device(NULL, Tk * F * b2);
  void* yp = to_device(NULL, Tk * d * b2);
  void* y = to_device(NULL, (size_t)T * d * b2);
  /* backward */
  float* dw = (float*)to_device(NULL, Tk * 4);
  float* w_sorted = (float*)to_device(NULL, Tk * 4);
  void* da = to_device(NULL, Tk * F * b2);
  void* dh = to_device(NULL, Tk * 2 * F * b2);
  void* dxp = to_device(NULL, Tk * d * b2);
  void* dx_e = to_device(NULL, (size_t)T * d * b2);
  void* dx = to_device(NULL, (size_t)T * d * b2);
  void* dlogits = to_device(NULL, (size_t)T * E * b2);
  float* dwr = (float*)to_device(NULL, (size_t)d * E * 4);
  float* dw1 = (float*)to_device(NULL, (size_t)E * d * 2 * F * 4);
  float* dw2 = (float*)to_device(NULL, (size_t)E * F * d * 4);
  size_t gws_bytes = moe_grouped_gemm_workspace_size(T, d, E, 1, MOE_BF16);
  const size_t g2 = moe_grouped_gemm_workspace_size((int)Tk, F, d, E, MOE_BF16);
  const size_t g1 = moe_grouped_gemm_workspace_size((int)Tk, d, 2 * F, E, MOE_BF16);
  if (g2 > gws_bytes) gws_bytes = g2;
  if (g1 > gws_bytes) gws_bytes = g1;
  void* gws = to_device(NULL, gws_bytes);

  unsigned int mask = 0, mask_bwd = 0;
  CHECK_MOE(moe_index_errors(&mask, 1, NULL)); /* start from a clear record */

  /* One stream (the null stream): every call only enqueues. */
  CHECK_MOE(moe_grouped_gemm_fwd(x, wr, router_off, T, d, E, 1, MOE_BF16, logits, MOE_F32,
                                 NULL, 0, NULL));
  CHECK_MOE(moe_route_topk(logits, NULL, T, E, k, 0, NULL, idx, w, probs, NULL));
  CHECK_MOE(moe_count_index(idx, T, k, E, counts, offsets, dest, src, ci_ws, ci_bytes, NULL));
  CHECK_MOE(moe_grouped_gemm_swiglu_fwd_gather(x, src, k, T, w1, offsets, (int)Tk, d, F, E,
                                               MOE_BF16, h, a, NULL));
  CHECK_MOE(moe_grouped_gemm_fwd(a, w2, offsets, (int)Tk, F, d, E, MOE_BF16, yp, MOE_BF16,
                                 NULL, 0, NULL));
  CHECK_MOE(moe_unpermute(yp, dest, w, T, k, d, MOE_BF16, y, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_MOE(moe_index_errors(&mask, 1, NULL));

  /* Backward of <y, dy>.  GEMM 2's backward reads dy through the row map
   * with the gate weight as a row scale; the SwiGLU backward writes the
   * scaled activation into a's buffer (a is not read again). */
  CHECK_MOE(moe_unpermute_bwd(dy, yp, dest, w, T, k, d, MOE_BF16, NULL, dw, NULL));
  CHECK_MOE(moe_gather_scale(w, src, (int)Tk, w_sorted, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd_scaled_gather(NULL, w2, dy, src, k, T, w_sorted, offsets,
                                               (int)Tk, F, d, E, MOE_BF16, da, NULL, gws,
                                               gws_bytes, NULL));
  CHECK_MOE(moe_act_bwd_scaled(h, da, w_sorted, (int)Tk, F, MOE_BF16, dh, a, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd_scaled_gather(a, NULL, dy, src, k, T, w_sorted, offsets,
                                               (int)Tk, F, d, E, MOE_BF16, NULL, dw2, gws,
                                               gws_bytes, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd(NULL, w1, dh, offsets, (int)Tk, d, 2 * F, E, MOE_BF16, dxp,
                                 NULL, NULL, gws, gws_bytes, NULL));
  CHECK_MOE(moe_unpermute(dxp, dest, NULL, T, k, d, MOE_BF16, dx_e, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd_gather(x, src, k, T, w1, dh, offsets, (int)Tk, d, 2 * F, E,
                                        MOE_BF16, NULL, NULL, dw1, gws, gws_bytes, NULL));
  CHECK_MOE(moe_route_topk_bwd(probs, idx, dw, T, E, k, 0, dlogits, MOE_BF16, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd(x, wr, dlogits, router_off, T, d, E, 1, MOE_BF16, dx, dx_e,
                                 NULL, gws, gws_bytes, NULL));
  CHECK_MOE(moe_grouped_gemm_bwd(x, wr, dlogits, router_off, T, d, E, 1, MOE_BF16, NULL, NULL,
                                 dwr, gws, gws_bytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_MOE(moe_index_errors(&mask_bwd, 1, NULL));

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) FAIL("cannot open %s", argv[2]);
  from_device(out, logits, (size_t)T * E * 4);
  from_device(out, idx, Tk * 4);
  from_device(out, w, Tk * 4);
  from_device(out, offsets, (size_t)(E + 1) * 4);
  from_device(out, y, (size_t)T * d * b2);
  from_device(out, dx, (size_t)T * d * b2);
  from_device(out, dwr, (size_t)d * E * 4);
  from_device(out, dw1, (size_t)E * d * 2 * F * 4);
  from_device(out, dw2, (size_t)E * F * d * 4);
  if (fwrite(&mask, sizeof mask, 1, out) != 1 || fwrite(&mask_bwd, sizeof mask_bwd, 1, out) != 1)
    FAIL("short write");
  fclose(out);

  void* bufs[] = {x,  wr, w1,       w2, dy,  router_off, logits, idx, w,       probs, counts,
                  offsets, dest, src, ci_ws, h, a, yp, y, dw, w_sorted, da, dh,
                  dxp, dx_e, dx, dlogits, dwr, dw1, dw2, gws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
  free(hx);
  free(hwr);
  free(hw1);
  free(hw2);
  free(hdy);
  printf("forward and backward ok: T=%d d=%d E=%d k=%d F=%d\n", T, d, E, k, F);
  return 0;
}
