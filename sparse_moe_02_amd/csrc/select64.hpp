// Binary64 ranking shared by the prefill router and the decode kernel: exact-product
// dot products, their error radii, and the selection of the top k experts with the
// lowest-index tie-break when the binary64 values alone cannot order them.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr double kU64 = 1.1102230246251565404e-16;   // 2^-53

// Binary64 dot products of x with up to G router rows (rows past n are skipped), by one
// wave; the token row is read once and the loads of all G rows are in flight together.
// For each row, lane `lane` takes the 8-element chunks c = lane + 64 i (ascending i) and
// sums its exact products sequentially; a butterfly over the wave gives every lane the
// same total.  Also returns sum |x_h w_h|.  Each product passes through at most seq + 6
// roundings with seq = 8*ceil(H/512).
template <int G>
__device__ void wave_dot64_n(const uint16_t *x, const uint16_t *const *w16, const float *const *w32, int n, int H,
                             int lane, double *l, double *a) {
  double s[G], sa[G];
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = sa[g] = 0.0;
  for (int c0 = lane; c0 < H / 8; c0 += 4 * kWave) {
    uint4 xv[4], wa[G][4], wb[G][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * kWave;
      const int cc = c < H / 8 ? c : lane;
      xv[u] = *(const uint4 *)(x + 8 * cc);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= n) break;
        if (w16) {
          wa[g][u] = *(const uint4 *)(w16[g] + 8 * cc);
        } else {
          wa[g][u] = *(const uint4 *)(w32[g] + 8 * cc);
          wb[g][u] = *(const uint4 *)(w32[g] + 8 * cc + 4);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c0 + u * kWave >= H / 8) break;
      const float xf[8] = {bf16_lo(xv[u].x), bf16_hi(xv[u].x), bf16_lo(xv[u].y), bf16_hi(xv[u].y),
                           bf16_lo(xv[u].z), bf16_hi(xv[u].z), bf16_lo(xv[u].w), bf16_hi(xv[u].w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= n) break;
        float wf[8];
        if (w16) {
          wf[0] = bf16_lo(wa[g][u].x); wf[1] = bf16_hi(wa[g][u].x); wf[2] = bf16_lo(wa[g][u].y);
          wf[3] = bf16_hi(wa[g][u].y); wf[4] = bf16_lo(wa[g][u].z); wf[5] = bf16_hi(wa[g][u].z);
          wf[6] = bf16_lo(wa[g][u].w); wf[7] = bf16_hi(wa[g][u].w);
        } else {
          wf[0] = __uint_as_float(wa[g][u].x); wf[1] = __uint_as_float(wa[g][u].y);
          wf[2] = __uint_as_float(wa[g][u].z); wf[3] = __uint_as_float(wa[g][u].w);
          wf[4] = __uint_as_float(wb[g][u].x); wf[5] = __uint_as_float(wb[g][u].y);
          wf[6] = __uint_as_float(wb[g][u].z); wf[7] = __uint_as_float(wb[g][u].w);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double p = (double)xf[i] * (double)wf[i];  // exact
          s[g] += p;
          sa[g] += fabs(p);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g >= n) break;
    l[g] = wave_sum_f64(s[g]);
    a[g] = wave_sum_f64(sa[g]);
  }
}

// Error radius of a binary64 logit (plus bias) summed in any order with at most `depth`
// additions on the path of every product, relative to the sequential ascending-h
// binary64 sum (plus bias), whose own error to the exact value is at most H roundings of
// sum|p|.  `a` is the computed sum |x_h w_h|.
__device__ __forceinline__ double radius64(double lb, double a, int H, int depth) {
  return ((double)depth + 2.0 + (double)H) * kU64 * a * 1.001 + 4.0 * kU64 * fabs(lb) + 1e-300;
}

// Additions on any path of wave_dot64_n's sum.
__device__ __forceinline__ int wave_dot64_depth(int H) { return 8 * ((H + 511) / 512) + 6; }

// Sequential ascending-h binary64 logit: the same arithmetic as the plain definition.
__device__ double seq_dot64(const uint16_t *x, const uint16_t *w16, const float *w32, int H) {
  double acc = 0.0;
  for (int h = 0; h < H; ++h) {
    const double w = w16 ? (double)bf16_to_f32(w16[h]) : (double)w32[h];
    acc = __builtin_fma((double)bf16_to_f32(x[h]), w, acc);  // product exact: fma == mul+add
  }
  return acc;
}

// Membership in the best r of n candidates (order: value descending, index ascending)
// from values v with error radius rad: state 1 = certainly in, 2 = certainly out,
// 0 = undecided.  Candidate j may outrank i if v_j + rad_j >= v_i - rad_i, and
// certainly outranks i if v_j - rad_j > v_i + rad_i.
__device__ void classify(const double *v, const double *rad, int n, int r, int *state, int tid,
                         int nthr) {
  for (int i = tid; i < n; i += nthr) {
    const double lo = v[i] - rad[i], hi = v[i] + rad[i];
    int poss = 0, cert = 0;
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      poss += (v[j] + rad[j] >= lo);
      cert += (v[j] - rad[j] > hi);
    }
    state[i] = (poss < r) ? 1 : (cert >= r ? 2 : 0);
  }
}

// Shared per-workgroup scratch of the binary64 selection.
struct Sel64 {
  double v[kMaxExperts];
  double rad[kMaxExperts];
  double gl[kMaxExperts];    // logit used for the gate of each expert
  int cand[kMaxExperts];     // candidate -> expert
  int state[kMaxExperts];
  int chosen[kMaxExperts];   // per expert: 1 if selected
  int n, nin;
};

// Resolve the candidates S.cand[0..S.n) for `r` remaining slots with binary64 logits
// already in S.v/S.rad; undecided ones are summed sequentially.  Marks S.chosen.
__device__ __attribute__((unused)) void resolve64(Sel64 &S, int r, const uint16_t *x, const uint16_t *w16,
                          const float *w32, const float *bias, int H, int tid, int nthr) {
  classify(S.v, S.rad, S.n, r, S.state, tid, nthr);
  __syncthreads();
  if (tid == 0) S.nin = 0;
  __syncthreads();
  for (int c = tid; c < S.n; c += nthr) {
    if (S.state[c] == 1) {
      S.chosen[S.cand[c]] = 1;
      atomicAdd(&S.nin, 1);
    } else if (S.state[c] == 0) {
      const int e = S.cand[c];
      double l = seq_dot64(x, w16 ? w16 + (size_t)e * H : nullptr, w32 ? w32 + (size_t)e * H : nullptr, H);
      if (bias) l += (double)bias[e];
      S.v[c] = l;  // exact canonical value
    }
  }
  __syncthreads();
  const int rr = r - S.nin;
  for (int c = tid; c < S.n; c += nthr) {
    if (S.state[c] != 0) continue;
    const int e = S.cand[c];
    int rank = 0;
    for (int j = 0; j < S.n; ++j)
      if (j != c && S.state[j] == 0)
        rank += (S.v[j] > S.v[c]) || (S.v[j] == S.v[c] && S.cand[j] < e);
    if (rank < rr) S.chosen[e] = 1;
    S.gl[e] = S.v[c];
  }
  __syncthreads();
}

}  // namespace

}  // namespace moe

namespace moe {

namespace {

// ------------------------------------------------------------------ wave-level re-ranking

// Scratch of one wave's re-ranking of one token (candidates in first-seen order).
struct WaveSel {
  double v[kMaxExperts];   // binary64 logit (+ bias) of candidate c
  float rad[kMaxExperts];  // its radius (rounded up to fp32)
  int16_t cand[kMaxExperts];  // candidate -> expert
  uint8_t state[kMaxExperts];  // 1 in, 2 out, 0 undecided
  int in_ids[kMaxTopK];        // chosen experts (any order)
  float in_l[kMaxTopK];    // the logit each chosen expert's gate uses
  int n_in;
};

// Orders this wave's LDS accesses before and after (lanes of one wave read each other's
// LDS writes).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int lane_rank(unsigned long long mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Re-rank one token with one wave.  `known_in(e)` / `known_out(e)` classify experts that
// the fp32 certificate already settles; every other expert is a candidate and gets a
// binary64 logit; candidates the binary64 radii cannot order are summed sequentially in
// ascending h (the plain definition's arithmetic, bit for bit).  Writes ids (ascending)
// and softmax gates, and returns the chosen ids (ascending) in W.in_ids[0..k).
template <class KnownIn, class KnownOut, class Fp32Logit>
__device__ void rerank_wave(WaveSel &W, KnownIn known_in, KnownOut known_out, Fp32Logit l32, int E, int k,
                            const uint16_t *xrow, const uint16_t *wr16, const float *wr32, const float *bias, int H,
                            int lane, int32_t *ids, float *gates, int32_t *dbg_ids, float *dbg_gates) {
  // 1. settled-in experts and the candidate list
  int n_in = 0, n_c = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    const bool valid = e < E;
    const bool in = valid && known_in(e);
    const bool cand = valid && !in && !known_out(e);
    const unsigned long long bi = __ballot(in), bc = __ballot(cand);
    if (in) {
      const int p = n_in + lane_rank(bi, lane);
      if (p < kMaxTopK) {
        W.in_ids[p] = e;
        W.in_l[p] = l32(e);
      }
    }
    if (cand) W.cand[n_c + lane_rank(bc, lane)] = (int16_t)e;
    n_in += __popcll(bi);
    n_c += __popcll(bc);
  }
  n_in = min(n_in, k);
  // 2. binary64 logits of the candidates, wave-wide dot products, kG rows at a time.  A
  // token that reaches this path has two candidates as a rule.  With kG = 4 the unrolled
  // code jumps over the unused rows' instructions at every chunk, and the path runs once
  // per launch on a workgroup, so each jump lands on code that is not in the instruction
  // cache; kG = 2 measured 2.5 us for this step against 4.1 us.
  constexpr int kG = 2;
  for (int c0 = 0; c0 < n_c; c0 += kG) {
    const int ng = min(kG, n_c - c0);
    const uint16_t *r16[kG];
    const float *r32[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const int e = W.cand[c0 + min(g, ng - 1)];
      r16[g] = wr16 ? wr16 + (size_t)e * H : nullptr;
      r32[g] = wr32 ? wr32 + (size_t)e * H : nullptr;
    }
    double l[kG], ab[kG];
    if (wr16)
      wave_dot64_n<kG>(xrow, r16, nullptr, ng, H, lane, l, ab);
    else
      wave_dot64_n<kG / 2>(xrow, nullptr, r32, min(ng, kG / 2), H, lane, l, ab);
    const int done = wr16 ? ng : min(ng, kG / 2);
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      if (g >= done) break;
      const int e = W.cand[c0 + g];
      double lv = l[g];
      if (bias) lv += (double)bias[e];
      if (lane == 0) {
        W.v[c0 + g] = lv;
        W.rad[c0 + g] = __double2float_ru(radius64(lv, ab[g], H, wave_dot64_depth(H)));
      }
    }
    if (!wr16) c0 -= kG - done;  // float32 rows go two at a time
  }
  wave_sync();
  // 3. membership among the candidates for the r remaining places
  const int r = k - n_in;
  for (int i = lane; i < n_c; i += kWave) {
    const double lo = W.v[i] - W.rad[i], hi = W.v[i] + W.rad[i];
    int poss = 0, cert = 0;
    for (int j = 0; j < n_c; ++j) {
      if (j == i) continue;
      poss += (W.v[j] + W.rad[j] >= lo);
      cert += (W.v[j] - W.rad[j] > hi);
    }
    W.state[i] = (uint8_t)((poss < r) ? 1 : (cert >= r ? 2 : 0));
  }
  wave_sync();
  // undecided candidates: exact canonical value, one lane each
  int n_cin = 0;
  for (int i0 = 0; i0 < n_c; i0 += kWave) {
    const int i = i0 + lane;
    const bool und = i < n_c && W.state[i] == 0;
    if (und) {
      const int e = W.cand[i];
      double l = seq_dot64(xrow, wr16 ? wr16 + (size_t)e * H : nullptr, wr32 ? wr32 + (size_t)e * H : nullptr, H);
      if (bias) l += (double)bias[e];
      W.v[i] = l;
    }
    n_cin += __popcll(__ballot(i < n_c && W.state[i] == 1));
  }
  wave_sync();
  const int rr = r - n_cin;  // places left for the undecided ones
  for (int i0 = 0; i0 < n_c; i0 += kWave) {
    const int i = i0 + lane;
    bool take = false;
    if (i < n_c) {
      if (W.state[i] == 1) {
        take = true;
      } else if (W.state[i] == 0) {
        int rank = 0;
        for (int j = 0; j < n_c; ++j)
          if (j != i && W.state[j] == 0) rank += (W.v[j] > W.v[i]) || (W.v[j] == W.v[i] && W.cand[j] < W.cand[i]);
        take = rank < rr;
      }
    }
    const unsigned long long bt = __ballot(take);
    if (take) {
      const int p = n_in + lane_rank(bt, lane);
      if (p < kMaxTopK) {
        W.in_ids[p] = W.cand[i];
        W.in_l[p] = (float)W.v[i];
      }
    }
    n_in += __popcll(bt);
  }
  wave_sync();
  // 4. ascending ids and softmax gates
  const int n = min(n_in, k);
  int my_e = 0x7fffffff;
  float my_l = -INFINITY;
  if (lane < n) {
    my_e = W.in_ids[lane];
    my_l = W.in_l[lane];
  }
  const float mx = wave_max(my_l);
  const float ex = lane < n ? __expf(my_l - mx) : 0.f;
  const float den = wave_sum(ex);
  int pos = 0;
  for (int j = 0; j < n; ++j) pos += __builtin_amdgcn_readlane(my_e, j) < my_e;
  wave_sync();
  if (lane < n) {
    const float g = ex / den;
    ids[pos] = my_e;
    gates[pos] = g;
    if (dbg_ids) dbg_ids[pos] = my_e;
    if (dbg_gates) dbg_gates[pos] = g;
    W.in_ids[pos] = my_e;
  }
  wave_sync();
}

}  // namespace

}  // namespace moe
