// Router: logits, top-k selection with lowest-index tie-break, softmax gates.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates three
// different workload shapes": the router scores every routed expert and keeps eight
// per token.  The selection is defined on exact logits (ties: lower index wins).
//
// Prefill: one workgroup per 32 tokens.  Logits and the bound sum_h |x_h w_eh| come
// from two bf16 MFMA chains with fp32 accumulation (bf16 x bf16 products are exact in
// fp32).  A token's fp32 ranking is certified when every chosen logit minus its error
// radius exceeds every other logit plus its radius; otherwise the token is re-ranked:
// undecided experts get binary64 logits (wave-parallel), and experts that even these
// cannot order are summed sequentially in ascending h in binary64, which reproduces the
// exact-product sequential sum bit for bit.
//
// Decode: one wave per expert computes binary64 logits; the last workgroup to finish
// (ticket counter) selects, falling back to sequential sums for undecided experts.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr float kU32 = 5.9604644775390625e-8f;       // 2^-24
constexpr double kU64 = 1.1102230246251565404e-16;   // 2^-53

// Binary64 dot product of x with one router row, by one wave.  Lane `lane` takes the
// 8-element chunks c = lane + 64 i (ascending i) and sums its exact products
// sequentially; a butterfly over the wave gives every lane the same total.  Also
// returns sum |x_h w_h|.  Each product passes through at most seq + 6 roundings with
// seq = 8*ceil(H/512).
__device__ void wave_dot64(const uint16_t *x, const uint16_t *w16, const float *w32, int H,
                           int lane, double &l, double &a) {
  double s = 0.0, sa = 0.0;
  for (int c = lane; c < H / 8; c += kWave) {
    const uint4 xv = *(const uint4 *)(x + 8 * c);
    float xf[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                   bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
    float wf[8];
    if (w16) {
      const uint4 wv = *(const uint4 *)(w16 + 8 * c);
      wf[0] = bf16_lo(wv.x); wf[1] = bf16_hi(wv.x); wf[2] = bf16_lo(wv.y); wf[3] = bf16_hi(wv.y);
      wf[4] = bf16_lo(wv.z); wf[5] = bf16_hi(wv.z); wf[6] = bf16_lo(wv.w); wf[7] = bf16_hi(wv.w);
    } else {
      const float4 w0 = *(const float4 *)(w32 + 8 * c);
      const float4 w1 = *(const float4 *)(w32 + 8 * c + 4);
      wf[0] = w0.x; wf[1] = w0.y; wf[2] = w0.z; wf[3] = w0.w;
      wf[4] = w1.x; wf[5] = w1.y; wf[6] = w1.z; wf[7] = w1.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double p = (double)xf[i] * (double)wf[i];  // exact
      s += p;
      sa += fabs(p);
    }
  }
  l = wave_sum_f64(s);
  a = wave_sum_f64(sa);
}

// Error radius of a wave_dot64 logit (plus bias) relative to the sequential
// ascending-h binary64 sum (plus bias), whose own error to the exact value is at most
// H roundings of sum|p|.
__device__ __forceinline__ double radius64(double lb, double a, int H) {
  const double seq = 8.0 * ((H + 511) / 512);
  return (seq + 8.0 + (double)H) * kU64 * a * 1.001 + 4.0 * kU64 * fabs(lb) + 1e-300;
}

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
  int list[kMaxTopK];
  int n, nin;
};

// Resolve the candidates S.cand[0..S.n) for `r` remaining slots with binary64 logits
// already in S.v/S.rad; undecided ones are summed sequentially.  Marks S.chosen.
__device__ void resolve64(Sel64 &S, int r, const uint16_t *x, const uint16_t *w16,
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

// Compact S.chosen (E experts) into ascending S.list and write ids/gates (softmax of
// S.gl over the chosen experts).
__device__ void emit_selection(Sel64 &S, int E, int k, int32_t *ids, float *gates, int32_t *dbg_ids,
                               float *dbg_gates, int tid, int nthr) {
  if (tid < k) S.list[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += nthr) {
    if (!S.chosen[e]) continue;
    int pos = 0;
    for (int j = 0; j < e; ++j) pos += S.chosen[j];
    if (pos < k) S.list[pos] = e;
  }
  __syncthreads();
  if (tid < k) {
    double mx = -INFINITY, den = 0.0;
    for (int j = 0; j < k; ++j) mx = fmax(mx, S.gl[S.list[j]]);
    for (int j = 0; j < k; ++j) den += exp(S.gl[S.list[j]] - mx);
    const int e = S.list[tid];
    const float g = (float)(exp(S.gl[e] - mx) / den);
    ids[tid] = e;
    gates[tid] = g;
    if (dbg_ids) dbg_ids[tid] = e;
    if (dbg_gates) dbg_gates[tid] = g;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------- prefill

__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
  __shared__ float s_l[kRouteTokens][kMaxExperts];   // fp32 logit (+bias)
  __shared__ float s_r[kRouteTokens][kMaxExperts];   // its error radius
  __shared__ int s_sel[kRouteTokens][kMaxTopK];      // chosen experts (any order)
  __shared__ int s_flag[kRouteTokens];
  __shared__ uint32_t s_mask[kMaxExperts];
  __shared__ Sel64 S;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, k = a.k;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);

  {  // the combine accumulator of these tokens starts at zero
    float4 *oa = (float4 *)(a.out_acc + (size_t)t0 * H);
    const int n4 = nt * H / 4;
    for (int i = tid; i < n4; i += 256) oa[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = tid; e < kMaxExperts; e += 256) s_mask[e] = 0;
  if (tid < kRouteTokens) s_flag[tid] = 0;

  if (a.wr16) {
    // 32 tokens x 32 experts per MFMA tile; wave wv takes expert tiles wv and wv+4.
    const int m = lane & 31, hf = lane >> 5;
    const int tok = t0 + min(m, nt - 1);
    const uint16_t *xr = a.x + (size_t)tok * H + 8 * hf;
    const int nct = (E + 31) / 32;
    const int ct0 = wv, ct1 = wv + 4;
    const bool has1 = ct1 < nct;
    if (ct0 < nct) {
      const uint16_t *w0 = a.wr16 + (size_t)min(ct0 * 32 + m, E - 1) * H + 8 * hf;
      const uint16_t *w1 = a.wr16 + (size_t)min(ct1 * 32 + m, E - 1) * H + 8 * hf;
      f32x16 acc0 = {}, acc1 = {}, abs0 = {}, abs1 = {};
      const u32x4 msk = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
#pragma unroll 4
      for (int kk = 0; kk < H; kk += 16) {
        const u32x4 av = *(const u32x4 *)(xr + kk);
        const u32x4 b0 = *(const u32x4 *)(w0 + kk);
        const u32x4 aa = av & msk;
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, b0), acc0, 0, 0, 0);
        abs0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aa), __builtin_bit_cast(bf16x8, (u32x4)(b0 & msk)), abs0, 0, 0, 0);
        if (has1) {
          const u32x4 b1 = *(const u32x4 *)(w1 + kk);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, b1), acc1, 0, 0, 0);
          abs1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aa), __builtin_bit_cast(bf16x8, (u32x4)(b1 & msk)), abs1, 0, 0, 0);
        }
      }
      // fp32 error of an MFMA chain of H/16 steps of 16 exact products: at most
      // (H/16 + 15) roundings of sum|p|; doubled for margin, plus the bias addition,
      // the sequential binary64 reference's own error and product underflow.
      const float c32 = 2.0f * (float)(H / 16 + 16) + 4.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && !has1) break;
        const int e = (t ? ct1 : ct0) * 32 + m;
        if (e >= E) continue;
        const float bb = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = 8 * (j >> 2) + 4 * hf + (j & 3);
          const float l = (t ? acc1[j] : acc0[j]) + bb;
          const float ab = (t ? abs1[j] : abs0[j]);
          s_l[row][e] = l;
          s_r[row][e] = c32 * kU32 * ab * 1.01f + 2.0f * kU32 * fabsf(l) + 1e-12f * ab + 1e-30f;
        }
      }
    }
  } else {
    // float32 router weights: no fp32 ranking; every expert is re-ranked in binary64.
    for (int i = tid; i < kRouteTokens * kMaxExperts; i += 256) {
      (&s_l[0][0])[i] = 0.0f;
      (&s_r[0][0])[i] = INFINITY;
    }
  }
  __syncthreads();

  // fp32 selection: wave wv takes tokens 8wv..8wv+7, eight lanes per token.
  {
    const int g = lane >> 3, q = lane & 7;
    const int m = wv * 8 + g;
    float lv[kMaxExperts / 8], rv[kMaxExperts / 8];
#pragma unroll
    for (int i = 0; i < kMaxExperts / 8; ++i) {
      const int e = q + 8 * i;
      lv[i] = e < E ? s_l[m][e] : -INFINITY;
      rv[i] = e < E ? s_r[m][e] : 0.0f;
    }
    uint32_t taken = 0;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxExperts / 8; ++i) {
        const int e = q + 8 * i;
        const bool ok = e < E && !((taken >> i) & 1u);
        if (ok && (lv[i] > bv || (lv[i] == bv && e < bi))) {
          bv = lv[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi < E && (bi & 7) == q) taken |= 1u << (bi >> 3);
      if (q == 0) s_sel[m][r] = bi < E ? bi : 0;
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 8; ++i) {
      const int e = q + 8 * i;
      if (e >= E) continue;
      if ((taken >> i) & 1u)
        mn = fminf(mn, lv[i] - rv[i]);
      else
        mx = fmaxf(mx, lv[i] + rv[i]);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const bool cert = mn > mx;  // false for NaN or infinite radius
    __syncthreads();
    if (m < nt && cert) {
      const float top = s_l[m][s_sel[m][0]];
      float ex[2] = {0.f, 0.f};
      int ee[2] = {0, 0};
      float den = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = q + 8 * u;
        if (r < k) {
          ee[u] = s_sel[m][r];
          ex[u] = __expf(s_l[m][ee[u]] - top);
          den += ex[u];
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) den += __shfl_xor(den, o);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = q + 8 * u;
        if (r >= k) continue;
        int pos = 0;
        for (int j = 0; j < k; ++j) pos += s_sel[m][j] < ee[u];
        const size_t o = (size_t)(t0 + m) * k + pos;
        const float gt = ex[u] / den;
        a.ids[o] = ee[u];
        a.gates[o] = gt;
        if (a.dbg_ids) a.dbg_ids[o] = ee[u];
        if (a.dbg_gates) a.dbg_gates[o] = gt;
      }
    } else if (m < nt && q == 0) {
      s_flag[m] = 1;
    }
  }
  __syncthreads();

  // binary64 re-ranking of the tokens the fp32 certificate did not settle
  int n_ref = 0;
  for (int m = 0; m < nt; ++m) {
    if (!s_flag[m]) continue;
    ++n_ref;
    const uint16_t *xrow = a.x + (size_t)(t0 + m) * H;
    for (int e = tid; e < E; e += 256) {
      S.v[e] = s_l[m][e];
      S.rad[e] = s_r[m][e];
      S.gl[e] = s_l[m][e];
      S.chosen[e] = 0;
    }
    __syncthreads();
    if (a.wr16) {
      classify(S.v, S.rad, E, k, S.state, tid, 256);
    } else {
      // no fp32 logits: every expert is a binary64 candidate
      for (int e = tid; e < E; e += 256) S.state[e] = 0;
    }
    if (tid == 0) S.n = 0;
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      if (S.state[e] == 1) S.chosen[e] = 1;
      if (S.state[e] == 0) S.cand[atomicAdd(&S.n, 1)] = e;
    }
    __syncthreads();
    int nin1 = 0;
    for (int e = 0; e < E; ++e) nin1 += S.chosen[e];
    // binary64 logits of the undecided experts, one wave each
    for (int c = wv; c < S.n; c += 4) {
      const int e = S.cand[c];
      double l, ab;
      wave_dot64(xrow, a.wr16 ? a.wr16 + (size_t)e * H : nullptr, a.wr32 ? a.wr32 + (size_t)e * H : nullptr, H,
                 lane, l, ab);
      if (a.bias) l += (double)a.bias[e];
      if (lane == 0) {
        S.v[c] = l;
        S.rad[c] = radius64(l, ab, H);
        S.gl[e] = l;
      }
    }
    __syncthreads();
    resolve64(S, k - nin1, xrow, a.wr16, a.wr32, a.bias, H, tid, 256);
    emit_selection(S, E, k, a.ids + (size_t)(t0 + m) * k, a.gates + (size_t)(t0 + m) * k,
                   a.dbg_ids ? a.dbg_ids + (size_t)(t0 + m) * k : nullptr,
                   a.dbg_gates ? a.dbg_gates + (size_t)(t0 + m) * k : nullptr, tid, 256);
    if (tid < k) s_sel[m][tid] = S.list[tid];
    __syncthreads();
  }

  // per-expert bit masks of this workgroup's tokens (histogram / rank source)
  for (int i = tid; i < nt * k; i += 256) {
    const int m = i / k, r = i - m * k;
    atomicOr(&s_mask[s_sel[m][r]], 1u << m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) a.tokmask[(size_t)blockIdx.x * E + e] = s_mask[e];
  if (tid == 0 && n_ref) atomicAdd(&a.ctrl->n_refined, n_ref);
}

// ---------------------------------------------------------------------------- decode

__global__ __launch_bounds__(64) void k_decode_route(DecodeArgs a) {
  __shared__ Sel64 S;
  __shared__ int s_last;
  const int lane = threadIdx.x;
  const int e = blockIdx.x, H = a.H, E = a.E, k = a.k;
  double l, ab;
  wave_dot64(a.x, a.wr16 ? a.wr16 + (size_t)e * H : nullptr, a.wr32 ? a.wr32 + (size_t)e * H : nullptr, H, lane, l,
             ab);
  if (a.bias) l += (double)a.bias[e];
  if (lane == 0) {
    a.l64[e] = l;
    a.a64[e] = radius64(l, ab, H);
    const int t = __hip_atomic_fetch_add(&a.ctrl->decode_ticket, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (t == E - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int i = lane; i < E; i += kWave) {
    S.v[i] = __hip_atomic_load(&a.l64[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.rad[i] = __hip_atomic_load(&a.a64[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.gl[i] = S.v[i];
    S.cand[i] = i;
    S.chosen[i] = 0;
  }
  if (lane == 0) S.n = E;
  __syncthreads();
  resolve64(S, k, a.x, a.wr16, a.wr32, a.bias, H, lane, kWave);
  emit_selection(S, E, k, a.ids, a.gates, a.dbg_ids, a.dbg_gates, lane, kWave);
  if (lane == 0) __hip_atomic_store(&a.ctrl->decode_ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void k_ctrl_init(Ctrl *c) {
  int *p = (int *)c;
  for (int i = threadIdx.x; i < (int)(sizeof(Ctrl) / sizeof(int)); i += blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(k_route, dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_route(const DecodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_decode_route, dim3(a.E), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ctrl_init(Ctrl *c, hipStream_t s) {
  hipLaunchKernelGGL(k_ctrl_init, dim3(1), dim3(64), 0, s, c);
  return hipGetLastError();
}

}  // namespace moe
