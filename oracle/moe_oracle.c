/*
 * moe_oracle.c -- plain, slow CPU oracle for the sparse MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library never
 * links, includes or calls it, and this file shares no code with it.
 *
 * Everything is computed in IEEE binary64 with plain loops in a fixed order.
 * What it computes is the plain definition of the layer described in
 * "Optimizing on-device inference for Apple Silicon":
 *   - section "Qwen creates three different workload shapes": a router scores
 *     every routed expert, each token goes to the top 8 of 256, and one shared
 *     expert processes every token;
 *   - section "Prefill > Dequantize weights during matmul": each weight is a
 *     4-bit integer code; each group of 64 weights carries a scale and a bias
 *     that reconstruct it (w = scale*code + bias);
 *   - section "Prefill > Keep expert routing on the GPU": a histogram counts
 *     assignments per expert, a prefix scan turns counts into start offsets and
 *     a scatter places every routed row in its expert's group;
 *   - section "Decode > Reduce intermediate and state traffic": the expert's two
 *     input projections feed a gated activation, and the output projection is
 *     weighted by the routing score and summed with the shared expert's result.
 * The pages leave the scoring rule, tie-break, activation and precision open;
 * the readings taken here are:
 *   - logits l[t][e] = sum_h x[t][h]*Wr[e][h] summed in ascending h in binary64
 *     (every product is exact in binary64), then + bias[e] if present;
 *   - selection: experts ordered by (logit descending, index ascending), the
 *     first k are chosen (equal logits: the lower index wins);
 *   - gates: softmax over the chosen logits (equal to a softmax over all experts
 *     renormalised over the chosen ones);
 *   - activation: SwiGLU, h = silu(gate) * up with silu(a) = a / (1 + exp(-a));
 *   - the shared expert is added with weight 1;
 *   - quantised layout: W[N][K], code of element k in bits 4*(k%8) of word
 *     q[n][k/8]; one scale/bias pair per 64 consecutive k, IEEE binary16 or
 *     bfloat16 (the pages' checkpoint stores them as bf16; the same section);
 *   - the shared expert's output is added with weight 1, or, when a gate vector
 *     w_sg [H] (bf16) is given, with weight sigmoid(x_t . w_sg) (section
 *     "Decode > Reduce intermediate and state traffic" fuses the shared
 *     expert's result into the output projection; a learned scalar gate on it
 *     is the optional form).
 *
 * Shapes: T tokens, H hidden, E routed experts, k chosen per token, I the
 * intermediate size.  Expert matrices are stacked over E+1 experts with the
 * shared expert at index E: gate/up [E+1][I][H], down [E+1][H][I].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16 bit pattern -> exact double (normal, subnormal, zero, inf). */
double oracle_fp16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man | 0x400), ex - 25);
  return sign ? -v : v;
}

/* bfloat16 bit pattern -> exact double. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static inline int code_at(const uint32_t *row_words, int64_t k) {
  return (int)((row_words[k >> 3] >> (4 * (k & 7))) & 0xfu);
}

static double qparam_to_double(uint16_t v, int qbf16) {
  return qbf16 ? oracle_bf16_to_double(v) : oracle_fp16_to_double(v);
}

/* w[n][k] = scale[n][k/64] * code(n,k) + bias[n][k/64], exact in binary64.  scale and
 * bias are binary16 bit patterns (qbf16 == 0) or bfloat16 ones (qbf16 != 0). */
void oracle_dequant(const uint32_t *q, const uint16_t *scale, const uint16_t *bias,
                    int64_t N, int64_t K, int qbf16, double *w) {
  const int64_t G = K / 64;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint32_t *qr = q + n * (K / 8);
    for (int64_t g = 0; g < G; ++g) {
      const double s = qparam_to_double(scale[n * G + g], qbf16);
      const double b = qparam_to_double(bias[n * G + g], qbf16);
      for (int64_t k = g * 64; k < g * 64 + 64; ++k) w[n * K + k] = s * (double)code_at(qr, k) + b;
    }
  }
}

/* Router: logits, top-k selection and gates for every token.
 *   x        [T][H] bf16 bits
 *   rw       [E][H] bf16 bits (rw_fp32 == 0) or float32 (rw_fp32 != 0)
 *   rb       [E] float32 or NULL
 * Outputs (any of logits/ranked may be NULL):
 *   logits   [T][E]   binary64 logits including the bias
 *   ids      [T][k]   chosen experts, ascending expert index
 *   gates    [T][k]   gate of ids[t][j]
 *   ranked   [T][k]   chosen experts in selection order (best first)
 * Returns 0, or -1 on bad sizes. */
int oracle_route(const uint16_t *x, int64_t T, int64_t H, int64_t E, int64_t k,
                 const void *rw, int rw_fp32, const float *rb, double *logits,
                 int32_t *ids, double *gates, int32_t *ranked) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return -1;
#pragma omp parallel
  {
    double *l = (double *)malloc(sizeof(double) * E);
    double *xd = (double *)malloc(sizeof(double) * H);
    char *taken = (char *)malloc(E);
    int32_t *rk = (int32_t *)malloc(sizeof(int32_t) * k);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t h = 0; h < H; ++h) xd[h] = oracle_bf16_to_double(x[t * H + h]);
      for (int64_t e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int64_t h = 0; h < H; ++h) {
          double w = rw_fp32 ? (double)((const float *)rw)[e * H + h]
                             : oracle_bf16_to_double(((const uint16_t *)rw)[e * H + h]);
          acc += xd[h] * w;
        }
        if (rb) acc += (double)rb[e];
        l[e] = acc;
        if (logits) logits[t * E + e] = acc;
      }
      /* selection by (logit descending, index ascending) */
      memset(taken, 0, E);
      for (int64_t r = 0; r < k; ++r) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
        taken[best] = 1;
        rk[r] = (int32_t)best;
      }
      if (ranked)
        for (int64_t r = 0; r < k; ++r) ranked[t * k + r] = rk[r];
      /* gates: softmax over the chosen logits; listed by ascending expert */
      double m = l[rk[0]], den = 0.0;
      for (int64_t e = 0; e < E; ++e)
        if (taken[e]) den += exp(l[e] - m);
      int64_t j = 0;
      for (int64_t e = 0; e < E; ++e)
        if (taken[e]) {
          ids[t * k + j] = (int32_t)e;
          gates[t * k + j] = exp(l[e] - m) / den;
          ++j;
        }
    }
    free(l);
    free(xd);
    free(taken);
    free(rk);
  }
  return 0;
}

/* Grouping: histogram over the chosen experts (bin E = the shared expert, which
 * every token visits), exclusive prefix scan, and the grouped row order: for
 * e = 0..E, the tokens that visit e in ascending token order.
 *   ids       [T][k] ascending per token
 *   counts    [E+1], offsets [E+2] (offsets[E+1] = T*(k+1))
 *   row_token [T*(k+1)]  token of each grouped row
 *   slot_row  [T][k+1]   grouped row of (token, j); j = k is the shared slot */
int oracle_group(const int32_t *ids, int64_t T, int64_t E, int64_t k, int32_t *counts,
                 int32_t *offsets, int32_t *row_token, int32_t *slot_row) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  for (int64_t e = 0; e <= E; ++e) counts[e] = 0;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = ids[t * k + j];
      if (e < 0 || e >= E) return -1;
      counts[e] += 1;
    }
    counts[E] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e <= E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int64_t e = 0; e <= E; ++e) {
    for (int64_t t = 0; t < T; ++t) {
      int64_t slot = -1;
      if (e == E)
        slot = k;
      else
        for (int64_t j = 0; j < k; ++j)
          if (ids[t * k + j] == e) slot = j;
      if (slot < 0) continue;
      row_token[pos] = (int32_t)t;
      slot_row[t * (k + 1) + slot] = (int32_t)pos;
      ++pos;
    }
  }
  return 0;
}

/* Experts and combine:
 *   out[t] = sum_{j<k} gates[t][j] * FFN_{ids[t][j]}(x_t) + c_t * FFN_E(x_t)
 *   FFN_e(v) = Wd_e * (silu(Wg_e v) .* (Wu_e v))
 *   c_t = 1, or sigmoid(sum_h x[t][h] * w_sg[h]) (ascending h, binary64) when
 *   shared_gate (bf16 [H]) is not NULL
 * Contributions are added to out[t] in ascending expert index, shared last.
 *   gate_q/up_q [E+1][I][H/8], gate_s/.. [E+1][I][H/64]
 *   down_q [E+1][H][I/8], down_s/.. [E+1][H][I/64]
 *   out [T][H] binary64 */
int oracle_experts(const uint16_t *x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                   const int32_t *ids, const double *gates, const uint32_t *gate_q,
                   const uint16_t *gate_s, const uint16_t *gate_b, const uint32_t *up_q,
                   const uint16_t *up_s, const uint16_t *up_b, const uint32_t *down_q,
                   const uint16_t *down_s, const uint16_t *down_b, int qbf16,
                   const uint16_t *shared_gate, double *out) {
  if (T < 0 || H <= 0 || I <= 0 || H % 64 || I % 64 || E <= 0 || k <= 0 || k > E) return -1;
  double *wg = (double *)malloc(sizeof(double) * I * H);
  double *wu = (double *)malloc(sizeof(double) * I * H);
  double *wd = (double *)malloc(sizeof(double) * H * I);
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (T > 0 ? T : 1));
  double *g = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
  if (!wg || !wu || !wd || !tok || !g) {
    free(wg); free(wu); free(wd); free(tok); free(g);
    return -2;
  }
  for (int64_t i = 0; i < T * H; ++i) out[i] = 0.0;
  for (int64_t e = 0; e <= E; ++e) {
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t) {
      if (e == E) {
        tok[n] = t;
        g[n] = 1.0;
        if (shared_gate) {
          double z = 0.0;
          for (int64_t h = 0; h < H; ++h)
            z += oracle_bf16_to_double(x[t * H + h]) * oracle_bf16_to_double(shared_gate[h]);
          g[n] = 1.0 / (1.0 + exp(-z));
        }
        ++n;
        continue;
      }
      for (int64_t j = 0; j < k; ++j)
        if (ids[t * k + j] == e) {
          tok[n] = t;
          g[n] = gates[t * k + j];
          ++n;
        }
    }
    if (n == 0) continue;
    oracle_dequant(gate_q + e * I * (H / 8), gate_s + e * I * (H / 64), gate_b + e * I * (H / 64), I, H, qbf16, wg);
    oracle_dequant(up_q + e * I * (H / 8), up_s + e * I * (H / 64), up_b + e * I * (H / 64), I, H, qbf16, wu);
    oracle_dequant(down_q + e * H * (I / 8), down_s + e * H * (I / 64), down_b + e * H * (I / 64), H, I, qbf16,
                   wd);
#pragma omp parallel
    {
      double *xd = (double *)malloc(sizeof(double) * H);
      double *hh = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n; ++r) {
        const int64_t t = tok[r];
        for (int64_t h = 0; h < H; ++h) xd[h] = oracle_bf16_to_double(x[t * H + h]);
        for (int64_t i = 0; i < I; ++i) {
          double a = 0.0, u = 0.0;
          for (int64_t h = 0; h < H; ++h) {
            a += wg[i * H + h] * xd[h];
            u += wu[i * H + h] * xd[h];
          }
          hh[i] = a / (1.0 + exp(-a)) * u;
        }
        for (int64_t o = 0; o < H; ++o) {
          double y = 0.0;
          for (int64_t i = 0; i < I; ++i) y += wd[o * I + i] * hh[i];
          out[t * H + o] += g[r] * y;
        }
      }
      free(xd);
      free(hh);
    }
  }
  free(wg);
  free(wu);
  free(wd);
  free(tok);
  free(g);
  return 0;
}
