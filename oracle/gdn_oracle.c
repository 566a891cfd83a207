/*
 * gdn_oracle.c -- plain, slow CPU oracle for the Gated DeltaNet prefill scan.
 *
 * TEST INFRASTRUCTURE ONLY (same rules as moe_oracle.c: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it; the HIP library never
 * links, includes or calls it).
 *
 * What it computes: section "Prefill > Keep recurrent state on chip" of
 * "Optimizing on-device inference for Apple Silicon" -- during prefill each Gated
 * DeltaNet layer scans the prompt in order and carries a recurrent state matrix
 * forward; the state and its gate are 32-bit floats, query and key activations
 * bfloat16.  The pages do not print the update; the reading taken is the gated
 * delta rule of Yang, Kautz and Hatamizadeh ("Gated Delta Networks: Improving
 * Mamba2 with Delta Rule", ICLR 2025), per value head h and token t:
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S [d_v][d_k] (one row per value channel: the pages' "column" of the state
 * that one SIMD group owns), k_t, q_t in R^{d_k}, v_t in R^{d_v}, scalars
 * alpha_t (decay, the gate) and beta_t (write strength).  Value head h reads key
 * head h / (n_vheads / n_kheads) (consecutive value heads share a key head).
 *
 * Everything is IEEE binary64 with plain loops: S (I - beta k k^T) is formed as
 * S - beta (S k) k^T with S k summed over ascending i, then scaled by alpha and
 * the rank-one write added, element by element; o = S_t q summed over ascending i.
 *
 * Layouts (row-major): q, k bf16 bits [T][n_kheads][d_k]; v bf16 bits
 * [T][n_vheads][d_v]; alpha, beta float32 [T][n_vheads]; state binary64
 * [n_vheads][d_v][d_k] (in: S_0, out: S_T); out binary64 [T][n_vheads][d_v].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int oracle_gdn_scan(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                    const float *beta, int64_t T, int64_t n_kheads, int64_t n_vheads, int64_t dk,
                    int64_t dv, double *state, double *out) {
  if (T < 0 || n_kheads < 1 || n_vheads < 1 || n_vheads % n_kheads != 0 || dk < 1 || dv < 1) return 1;
  const int64_t group = n_vheads / n_kheads;
  double *kt = malloc(sizeof(double) * (size_t)dk);
  double *qt = malloc(sizeof(double) * (size_t)dk);
  double *sk = malloc(sizeof(double) * (size_t)dv);
  if (!kt || !qt || !sk) {
    free(kt);
    free(qt);
    free(sk);
    return 2;
  }
  for (int64_t h = 0; h < n_vheads; ++h) {
    const int64_t kh = h / group;
    double *S = state + h * dv * dk;
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t i = 0; i < dk; ++i) {
        kt[i] = bf16_bits_to_double(k[(t * n_kheads + kh) * dk + i]);
        qt[i] = bf16_bits_to_double(q[(t * n_kheads + kh) * dk + i]);
      }
      const double a = alpha[t * n_vheads + h], b = beta[t * n_vheads + h];
      /* S_{t-1} k_t */
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += S[j * dk + i] * kt[i];
        sk[j] = acc;
      }
      /* S_t = alpha (S_{t-1} - beta (S_{t-1} k) k^T) + beta v k^T */
      for (int64_t j = 0; j < dv; ++j) {
        const double vj = bf16_bits_to_double(v[(t * n_vheads + h) * dv + j]);
        for (int64_t i = 0; i < dk; ++i)
          S[j * dk + i] = a * (S[j * dk + i] - b * sk[j] * kt[i]) + b * vj * kt[i];
      }
      /* o_t = S_t q_t */
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += S[j * dk + i] * qt[i];
        out[(t * n_vheads + h) * dv + j] = acc;
      }
    }
  }
  free(kt);
  free(qt);
  free(sk);
  return 0;
}
