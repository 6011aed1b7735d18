/* A plain C99 caller of the device path: device buffers from the HIP runtime's C
 * API, rotattn_quantize_qk then rotattn_int4_attention through the C ABI, on the
 * tiny shape (B 1, H 2, grid 2x4x4, D 64 split 24/20/20, blocks of 16, Half
 * rotation), checked against the CPU oracle's C entry points: INT4 codes and scales
 * bit-exact, the output within max-abs 2e-3.  Built and run by
 * tests/test_gpu_parity.py.  Exit status 0 when every check holds, else the number
 * of the first failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rotattn.h"

/* the oracle's C entry points (test infrastructure) */
void orc_rope_table(const int32_t* shp, int32_t rot, double base, float* out);
int64_t orc_table_entries(const int32_t* shp);
void orc_quantize(const int32_t* shp, int32_t rot, const float* tab, int32_t smooth_k, const float* q,
                  const float* k, const float* v, int8_t* qc, float* qs, int8_t* kc, float* ks, int8_t* vc,
                  float* vs, int32_t* vcol, float* q_rot, float* k_rot, float* k_mu);
void orc_attention(const int32_t* shp, const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                   const int8_t* vc, const float* vs, const int64_t* rows, int64_t n_rows, double* out,
                   int32_t* a_qk, int8_t* pcode, int32_t* a_pv, float* m_out, double* l_out);

#define CHECK(c, n)  \
  do {               \
    if (!(c)) {      \
      fprintf(stderr, "check %d failed: %s\n", n, #c); \
      return n;      \
    }                \
  } while (0)

static uint32_t lcg_state = 12345u;
static float uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) / 8388608.0f - 1.0f;
}
static int nib(const uint8_t* p, int64_t i) { /* signed nibble i (low nibble first) */
  const int v = (p[i >> 1] >> (4 * (int)(i & 1))) & 15;
  return v >= 8 ? v - 16 : v;
}

int main(void) {
  const rotattn_shape s = {1, 2, 2, 4, 4, 64, 24, 20, 20, 16, 16};
  const int32_t shp[11] = {1, 2, 2, 4, 4, 64, 24, 20, 20, 16, 16};
  const int64_t BH = 2, N = 32, D = 64, Np = rotattn_padded_tokens(&s);
  const int64_t nqb = N / 16, nsc = Np / 16;
  const size_t nin = (size_t)(BH * N * D);
  float *q = malloc(nin * 4), *k = malloc(nin * 4), *v = malloc(nin * 4);
  size_t i;
  CHECK(Np == 256, 1);
  for (i = 0; i < nin; ++i) {
    q[i] = 3.0f * uniform();
    k[i] = 3.0f * uniform();
    v[i] = uniform();
  }
  /* the library's RoPE table and buffers */
  const size_t nt = rotattn_rope_table_floats(&s);
  float* tab = malloc(nt * 4);
  CHECK(rotattn_build_rope_table(&s, ROTATTN_ROT_HALF, 10000.0, tab) == ROTATTN_OK, 2);
  void *dq, *dk, *dv, *dtab, *dqc, *dqs, *dkc, *dks, *dvc, *dvs, *dws, *dout, *daw;
  const size_t ncode = (size_t)(BH * Np * D / 2), wsq = rotattn_quantize_qk_workspace(&s),
               wsa = rotattn_int4_attention_workspace(&s);
  CHECK(hipMalloc(&dq, nin * 4) == hipSuccess && hipMalloc(&dk, nin * 4) == hipSuccess &&
            hipMalloc(&dv, nin * 4) == hipSuccess && hipMalloc(&dtab, nt * 4) == hipSuccess &&
            hipMalloc(&dqc, ncode) == hipSuccess && hipMalloc(&dkc, ncode) == hipSuccess &&
            hipMalloc(&dvc, ncode) == hipSuccess && hipMalloc(&dqs, BH * nsc * 4) == hipSuccess &&
            hipMalloc(&dks, BH * nsc * 4) == hipSuccess && hipMalloc(&dvs, BH * D * 4) == hipSuccess &&
            hipMalloc(&dws, wsq) == hipSuccess && hipMalloc(&daw, wsa) == hipSuccess &&
            hipMalloc(&dout, nin * 4) == hipSuccess,
        3);
  CHECK(hipMemcpy(dq, q, nin * 4, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dk, k, nin * 4, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dv, v, nin * 4, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dtab, tab, nt * 4, hipMemcpyHostToDevice) == hipSuccess,
        4);
  CHECK(rotattn_quantize_qk(&s, ROTATTN_ROT_HALF, ROTATTN_F32, dq, dk, dv, (const float*)dtab, 1, (uint8_t*)dqc,
                            (float*)dqs, (uint8_t*)dkc, (float*)dks, (uint8_t*)dvc, (float*)dvs, NULL, dws, wsq,
                            NULL) == ROTATTN_OK,
        5);
  CHECK(rotattn_int4_attention(&s, (const uint8_t*)dqc, (const float*)dqs, (const uint8_t*)dkc,
                               (const float*)dks, (const uint8_t*)dvc, (const float*)dvs, NULL, 0, ROTATTN_F32,
                               dout, NULL, daw, wsa, NULL) == ROTATTN_OK,
        6);
  CHECK(hipDeviceSynchronize() == hipSuccess, 7);
  uint8_t *qc = malloc(ncode), *kc = malloc(ncode);
  float *qs = malloc(BH * nsc * 4), *ks = malloc(BH * nsc * 4), *out = malloc(nin * 4);
  CHECK(hipMemcpy(qc, dqc, ncode, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(kc, dkc, ncode, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(qs, dqs, BH * nsc * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(ks, dks, BH * nsc * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(out, dout, nin * 4, hipMemcpyDeviceToHost) == hipSuccess,
        8);
  /* the oracle, from the same inputs */
  const int64_t ne = orc_table_entries(shp);
  float* otab = malloc((size_t)ne * 4);
  orc_rope_table(shp, ROTATTN_ROT_HALF, 10000.0, otab);
  int8_t *oqc = malloc(nin), *okc = malloc(nin), *ovc = malloc(nin);
  float *oqs = malloc(BH * nqb * 4), *oks = malloc(BH * nqb * 4), *ovs = malloc(BH * D * 4);
  int32_t* ovcol = malloc(BH * (N / 16) * D * 4);
  orc_quantize(shp, ROTATTN_ROT_HALF, otab, 1, q, k, v, oqc, oqs, okc, oks, ovc, ovs, ovcol, NULL, NULL, NULL);
  int64_t bh, n, d, mism = 0;
  for (bh = 0; bh < BH; ++bh)
    for (n = 0; n < N; ++n)
      for (d = 0; d < D; ++d) {
        const int64_t src = ((bh * Np) + n) * D + d, ref = (bh * N + n) * D + d;
        mism += nib(qc, src) != oqc[ref];
        mism += nib(kc, src) != okc[ref];
      }
  CHECK(mism == 0, 9);
  for (bh = 0; bh < BH; ++bh)
    for (n = 0; n < nqb; ++n) {
      CHECK(memcmp(&qs[bh * nsc + n], &oqs[bh * nqb + n], 4) == 0, 10);
      CHECK(memcmp(&ks[bh * nsc + n], &oks[bh * nqb + n], 4) == 0, 11);
    }
  int64_t* rows = malloc(BH * N * 8);
  double* oo = malloc(nin * 8);
  for (n = 0; n < BH * N; ++n) rows[n] = n;
  orc_attention(shp, oqc, oqs, okc, oks, ovc, ovs, rows, BH * N, oo, NULL, NULL, NULL, NULL, NULL);
  double err = 0.0;
  for (i = 0; i < nin; ++i) err = fmax(err, fabs((double)out[i] - oo[i]));
  CHECK(err <= 2e-3, 12);
  printf("c device abi ok, max abs %.3g\n", err);
  return 0;
}
