/* The library driven end to end from plain C on the GPU, with no Python or
 * torch in the process: device buffers come from the HIP runtime directly,
 * one chunked forward (bf16, two sequences of 130 tokens: two full chunks
 * and a ragged one, with an initial state) runs on the null stream, then one
 * decode step continues from its final state. Both are checked against the
 * fp64 oracle (oracle/liboracle.so) with the bf16 bar: max|gpu - oracle| <=
 * 1e-2 * max|oracle| for the outputs and the states. Exit status 0 and a
 * final "ok" line on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gla.h"

/* the oracle's C entry points (oracle/gla_oracle.c) */
int oracle_gla_varlen(int N, const int64_t *cu, int H, int dk, int dv, const float *q,
                      const float *k, const float *v, const float *decay, double scale,
                      const double *s0, double *o, double *s_final, int nthreads);
int oracle_gla_decode(int N, int H, int dk, int dv, const float *q, const float *k,
                      const float *v, const float *decay, double scale, double *state,
                      double *o, int nthreads);

enum { B = 2, T = 130, H = 2, DK = 96, DV = 192 };

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      printf("HIP error %d at line %d\n", (int)e_, __LINE__);          \
      exit(1);                                                         \
    }                                                                  \
  } while (0)

/* seeded inputs: xorshift64* uniforms, Box-Muller normals */
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return ((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(void) {
  const double u = uniform01() + 1e-300, w = uniform01();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w));
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t bf16_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

/* bf16 inputs: the bits for the GPU, their exact fp32 values for the oracle */
static void draw(size_t n, float mult, uint16_t *bits, float *vals) {
  for (size_t i = 0; i < n; ++i) {
    bits[i] = bf16_bits(normal() * mult);
    vals[i] = bf16_value(bits[i]);
  }
}

static double rel_err_bf16(const uint16_t *got, const double *ref, size_t n) {
  double e = 0.0, m = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double d = fabs((double)bf16_value(got[i]) - ref[i]);
    if (d > e || d != d) e = d;
    if (fabs(ref[i]) > m) m = fabs(ref[i]);
  }
  return e / m;
}
static double rel_err_f32(const float *got, const double *ref, size_t n) {
  double e = 0.0, m = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double d = fabs((double)got[i] - ref[i]);
    if (d > e || d != d) e = d;
    if (fabs(ref[i]) > m) m = fabs(ref[i]);
  }
  return e / m;
}

int main(void) {
  const size_t nq = (size_t)B * T * H * DK, nv = (size_t)B * T * H * DV;
  const size_t ns = (size_t)B * H * DK * DV;
  const float qk_mult = (float)(1.0 / sqrt((double)DK));
  const float decay[H] = {0.96875f, 0.99609375f};
  uint16_t *qb = malloc(nq * 2), *kb = malloc(nq * 2), *vb = malloc(nv * 2), *ob = malloc(nv * 2);
  float *qf = malloc(nq * 4), *kf = malloc(nq * 4), *vf = malloc(nv * 4);
  float *s0 = malloc(ns * 4), *sf = malloc(ns * 4);
  double *s0d = malloc(ns * 8), *o_ref = malloc(nv * 8), *s_ref = malloc(ns * 8);
  if (!qb || !kb || !vb || !ob || !qf || !kf || !vf || !s0 || !sf || !s0d || !o_ref || !s_ref)
    return 1;
  draw(nq, qk_mult, qb, qf);
  draw(nq, qk_mult, kb, kf);
  draw(nv, 1.0f, vb, vf);
  for (size_t i = 0; i < ns; ++i) {
    s0[i] = normal() * 0.1f;
    s0d[i] = s0[i];
  }

  /* device buffers straight from the HIP runtime */
  void *dq, *dk, *dv, *dout, *ds0, *dsf, *ws = NULL;
  HIP_OK(hipMalloc(&dq, nq * 2));
  HIP_OK(hipMalloc(&dk, nq * 2));
  HIP_OK(hipMalloc(&dv, nv * 2));
  HIP_OK(hipMalloc(&dout, nv * 2));
  HIP_OK(hipMalloc(&ds0, ns * 4));
  HIP_OK(hipMalloc(&dsf, ns * 4));
  HIP_OK(hipMemcpy(dq, qb, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, kb, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, vb, nv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ds0, s0, ns * 4, hipMemcpyHostToDevice));
  const size_t wsb = gla_chunk_fwd_workspace_bytes(GLA_BF16, B, T, H, DK, DV, 0);
  if (wsb) HIP_OK(hipMalloc(&ws, wsb));

  gla_status st = gla_chunk_fwd(GLA_BF16, B, T, H, DK, DV, 0, dq, dk, dv, decay, 1.0f,
                                (const float *)ds0, dout, (float *)dsf, ws, wsb, NULL);
  if (st != GLA_OK) {
    printf("gla_chunk_fwd: %s\n", gla_status_str(st));
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(ob, dout, nv * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(sf, dsf, ns * 4, hipMemcpyDeviceToHost));

  int64_t cu[B + 1];
  for (int n = 0; n <= B; ++n) cu[n] = (int64_t)n * T;
  if (oracle_gla_varlen(B, cu, H, DK, DV, qf, kf, vf, decay, 1.0, s0d, o_ref, s_ref, 0) != 0)
    return 1;
  const double eo = rel_err_bf16(ob, o_ref, nv), es = rel_err_f32(sf, s_ref, ns);
  printf("forward: o %.2e  S_final %.2e\n", eo, es);

  /* one decode step on the GPU's final state (in place), one token per
     sequence; the oracle starts from the same fp32 state */
  const size_t tq = (size_t)B * H * DK, tv = (size_t)B * H * DV;
  uint16_t tqb[B * H * DK], tkb[B * H * DK], tvb[B * H * DV], tob[B * H * DV];
  float tqf[B * H * DK], tkf[B * H * DK], tvf[B * H * DV];
  double to_ref[B * H * DV];
  draw(tq, qk_mult, tqb, tqf);
  draw(tq, qk_mult, tkb, tkf);
  draw(tv, 1.0f, tvb, tvf);
  HIP_OK(hipMemcpy(dq, tqb, tq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, tkb, tq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, tvb, tv * 2, hipMemcpyHostToDevice));
  st = gla_decode_step(GLA_BF16, B, H, DK, DV, dq, dk, dv, decay, 1.0f, (float *)dsf, dout,
                       NULL);
  if (st != GLA_OK) {
    printf("gla_decode_step: %s\n", gla_status_str(st));
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(tob, dout, tv * 2, hipMemcpyDeviceToHost));
  float *sf2 = malloc(ns * 4);
  if (!sf2) return 1;
  HIP_OK(hipMemcpy(sf2, dsf, ns * 4, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < ns; ++i) s_ref[i] = sf[i];
  if (oracle_gla_decode(B, H, DK, DV, tqf, tkf, tvf, decay, 1.0, s_ref, to_ref, 0) != 0)
    return 1;
  const double edo = rel_err_bf16(tob, to_ref, tv), eds = rel_err_f32(sf2, s_ref, ns);
  printf("decode: o %.2e  state %.2e\n", edo, eds);

  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(ds0));
  HIP_OK(hipFree(dsf));
  if (ws) HIP_OK(hipFree(ws));
  if (!(eo <= 1e-2 && es <= 1e-2 && edo <= 1e-2 && eds <= 1e-2)) {
    printf("FAILED: above the 1e-2 bar\n");
    return 1;
  }
  printf("ok\n");
  return 0;
}
