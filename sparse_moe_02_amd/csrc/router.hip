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
  float ex[kMaxTopK];
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

// Compact the chosen experts into ascending S.list and write ids/gates (softmax of S.gl
// over them).  Experts are gathered unordered, then each of the k entries finds its
// rank among the k.
__device__ void emit_selection(Sel64 &S, int E, int k, int32_t *ids, float *gates, int32_t *dbg_ids,
                               float *dbg_gates, int tid, int nthr) {
  if (tid == 0) S.nin = 0;
  if (tid < kMaxTopK) S.list[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += nthr)
    if (S.chosen[e]) {
      const int at = atomicAdd(&S.nin, 1);
      if (at < kMaxTopK) S.cand[at] = e;
    }
  __syncthreads();
  const int n = min(S.nin, k);
  if (tid < n) {
    const int e = S.cand[tid];
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += S.cand[j] < e;
    S.list[pos] = e;
  }
  __syncthreads();
  if (tid < k) {  // each chosen expert's exponential once
    double mx = -INFINITY;
    for (int j = 0; j < k; ++j) mx = fmax(mx, S.gl[S.list[j]]);
    S.ex[tid] = __expf((float)(S.gl[S.list[tid]] - mx));
  }
  __syncthreads();
  if (tid < k) {
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += S.ex[j];
    const int e = S.list[tid];
    const float g = S.ex[tid] / den;
    ids[tid] = e;
    gates[tid] = g;
    if (dbg_ids) dbg_ids[tid] = e;
    if (dbg_gates) dbg_gates[tid] = g;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------- prefill

constexpr int kRouteThreads = 512;   // 8 waves: wave w owns experts 32w..32w+31
constexpr int kKC = 256;             // k per staged chunk of x
constexpr int kXRow = kKC * 2;       // bytes per staged row (32 slots of 16 B)

// swizzled position of 16-byte slot `slot` of staged row `r`
__device__ __forceinline__ int xoff(int r, int slot) { return r * kXRow + ((slot ^ (r & 15)) << 4); }

__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  __shared__ float s_l[kRouteTokens][kMaxExperts];   // fp32 logit (+bias)
  __shared__ float s_r[kRouteTokens][kMaxExperts];   // its error radius
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kRouteTokens * kXRow];
  __shared__ int s_sel[kRouteTokens][kMaxTopK];      // chosen experts (rank order)
  __shared__ float s_min_in[kRouteTokens], s_max_out[kRouteTokens];
  __shared__ int s_flag[kRouteTokens];
  __shared__ uint32_t s_mask[kMaxExperts];
  __shared__ Sel64 S;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, k = a.k;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);

  for (int e = tid; e < kMaxExperts; e += kRouteThreads) s_mask[e] = 0;
  if (tid < kRouteTokens) s_flag[tid] = 0;

  if (a.wr16) {
    const int m = lane & 31, hf = lane >> 5;
    const int nct = (E + 31) / 32;
    const bool active = wv < nct;
    const uint16_t *wrow = a.wr16 + (size_t)min(wv * 32 + m, E - 1) * H + 8 * hf;
    // x chunk loader: wave-load j fills staged rows 2j, 2j+1; lane L -> row 2j+L/32,
    // physical slot L%32 holding logical slot (L%32) ^ (row & 15)
    const int xr0 = 2 * wv + (lane >> 5), xr1 = xr0 + 16;
    const uint16_t *xg0 = a.x + (size_t)(t0 + min(xr0, nt - 1)) * H + 8 * ((lane & 31) ^ (xr0 & 15));
    const uint16_t *xg1 = a.x + (size_t)(t0 + min(xr1, nt - 1)) * H + 8 * ((lane & 31) ^ (xr1 & 15));
    auto load_x = [&](int c, int buf) {
      __builtin_amdgcn_global_load_lds((const void *)(xg0 + c * kKC),
                                       (__attribute__((address_space(3))) void *)(s_x[buf] + wv * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(xg1 + c * kKC),
                                       (__attribute__((address_space(3))) void *)(s_x[buf] + (wv + 8) * 1024), 16, 0,
                                       0);
    };
    u32x4 w0[kKC / 16], w1[kKC / 16];
    auto load_w = [&](int c, u32x4(&dst)[kKC / 16]) {
#pragma unroll
      for (int s2 = 0; s2 < kKC / 16; ++s2) dst[s2] = *(const u32x4 *)(wrow + c * kKC + 16 * s2);
    };
    const int nch = H / kKC;
    f32x16 acc = {}, aab = {};
    const u32x4 msk = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
    auto compute = [&](int buf, const u32x4(&wb)[kKC / 16]) {
#pragma unroll
      for (int s2 = 0; s2 < kKC / 16; ++s2) {
        const u32x4 av = *(const u32x4 *)(s_x[buf] + xoff(m, 2 * s2 + hf));
        const u32x4 bv = wb[s2];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
        aab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, (u32x4)(av & msk)),
                                                      __builtin_bit_cast(bf16x8, (u32x4)(bv & msk)), aab, 0, 0, 0);
      }
    };
    // two-stage pipeline: chunk c+1 (x into LDS, router rows into registers) is in
    // flight while chunk c is multiplied
    load_x(0, 0);
    if (active) load_w(0, w0);
    for (int c = 0; c < nch; c += 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c + 1 < nch) {
        load_x(c + 1, 1);
        if (active) load_w(c + 1, w1);
      }
      if (active) compute(0, w0);
      if (c + 1 >= nch) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c + 2 < nch) {
        load_x(c + 2, 0);
        if (active) load_w(c + 2, w0);
      }
      if (active) compute(1, w1);
    }
    if (active) {
      // fp32 error of an MFMA chain of H/16 steps of 16 exact products: at most
      // (H/16 + 15) roundings of sum|p|; doubled for margin, plus the bias addition,
      // the sequential binary64 reference's own error and product underflow.
      const float c32 = 2.0f * (float)(H / 16 + 16) + 4.0f;
      const int e = wv * 32 + m;
      if (e < E) {
        const float bb = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = 8 * (j >> 2) + 4 * hf + (j & 3);
          const float l = acc[j] + bb;
          s_l[row][e] = l;
          s_r[row][e] = c32 * kU32 * aab[j] * 1.01f + 2.0f * kU32 * fabsf(l) + 1e-12f * aab[j] + 1e-30f;
        }
      }
    }
  } else {
    // float32 router weights: no fp32 ranking; every expert is re-ranked in binary64.
    for (int i = tid; i < kRouteTokens * kMaxExperts; i += kRouteThreads) {
      (&s_l[0][0])[i] = 0.0f;
      (&s_r[0][0])[i] = INFINITY;
    }
  }
  __syncthreads();

  // fp32 selection: wave wv takes tokens 4wv..4wv+3, sixteen lanes per token.
  {
    const int g = lane >> 4, q = lane & 15;
    const int m = wv * 4 + g;
    constexpr int NV = kMaxExperts / 16;
    float lv[NV], rv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 16 * i;
      lv[i] = e < E ? s_l[m][e] : -INFINITY;
      rv[i] = e < E ? s_r[m][e] : 0.0f;
    }
    uint32_t taken = 0;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = q + 16 * i;
        if (e < E && !((taken >> i) & 1u) && (lv[i] > bv || (lv[i] == bv && e < bi))) {
          bv = lv[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi < E && (bi & 15) == q) taken |= 1u << (bi >> 4);
      if (q == 0) s_sel[m][r] = bi < E ? bi : 0;
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 16 * i;
      if (e >= E) continue;
      if ((taken >> i) & 1u)
        mn = fminf(mn, lv[i] - rv[i]);
      else
        mx = fmaxf(mx, lv[i] + rv[i]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const bool cert = mn > mx;  // false for NaN or an infinite radius
    if (q == 0) {
      s_min_in[m] = mn;
      s_max_out[m] = mx;
    }
    __syncthreads();
    if (m < nt && cert) {
      const float top = s_l[m][s_sel[m][0]];
      if (q < k) {
        const int e = s_sel[m][q];
        float ex = __expf(s_l[m][e] - top), den = 0.f;
        for (int j = 0; j < k; ++j) den += __expf(s_l[m][s_sel[m][j]] - top);
        int pos = 0;
        for (int j = 0; j < k; ++j) pos += s_sel[m][j] < e;
        const size_t o = (size_t)(t0 + m) * k + pos;
        const float gt = ex / den;
        a.ids[o] = e;
        a.gates[o] = gt;
        if (a.dbg_ids) a.dbg_ids[o] = e;
        if (a.dbg_gates) a.dbg_gates[o] = gt;
      }
    } else if (m < nt && q == 0) {
      s_flag[m] = 1;
    }
  }
  __syncthreads();

  // re-ranking of the tokens the fp32 certificate did not settle.  With S~ the fp32
  // top-k, lo = min over S~ of (l - r) and hi = max outside of (l + r): a chosen expert
  // with l - r > hi is in for sure, an outside one with l + r < lo is out for sure; the
  // rest get binary64 logits and are resolved in resolve64.
  int n_ref = 0;
  for (int m = 0; m < nt; ++m) {
    if (!s_flag[m]) continue;
    ++n_ref;
    const uint16_t *xrow = a.x + (size_t)(t0 + m) * H;
    const float lo = s_min_in[m], hi = s_max_out[m];
    if (tid == 0) S.n = 0;
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) {
      S.gl[e] = s_l[m][e];
      S.chosen[e] = 0;
      bool in_sel = false;
      for (int j = 0; j < k; ++j) in_sel |= s_sel[m][j] == e;
      const float L = s_l[m][e] - s_r[m][e], U = s_l[m][e] + s_r[m][e];
      const bool sure_in = a.wr16 && in_sel && L > hi;
      const bool sure_out = a.wr16 && !in_sel && U < lo;
      if (sure_in) S.chosen[e] = 1;
      if (!sure_in && !sure_out) S.cand[atomicAdd(&S.n, 1)] = e;
    }
    __syncthreads();
    int nin1 = 0;
    for (int j = 0; j < k; ++j) nin1 += S.chosen[s_sel[m][j]];
    for (int c = wv; c < S.n; c += kRouteThreads / kWave) {
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
    resolve64(S, k - nin1, xrow, a.wr16, a.wr32, a.bias, H, tid, kRouteThreads);
    emit_selection(S, E, k, a.ids + (size_t)(t0 + m) * k, a.gates + (size_t)(t0 + m) * k,
                   a.dbg_ids ? a.dbg_ids + (size_t)(t0 + m) * k : nullptr,
                   a.dbg_gates ? a.dbg_gates + (size_t)(t0 + m) * k : nullptr, tid, kRouteThreads);
    if (tid < k) s_sel[m][tid] = S.list[tid];
    __syncthreads();
  }

  // per-expert bit masks of this workgroup's tokens (histogram / rank source)
  for (int i = tid; i < nt * k; i += kRouteThreads) {
    const int m = i / k, r = i - m * k;
    atomicOr(&s_mask[s_sel[m][r]], 1u << m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) a.tokmask[(size_t)blockIdx.x * E + e] = s_mask[e];
  if (tid == 0 && n_ref) atomicAdd(&a.ctrl->n_refined, n_ref);
}

// ---------------------------------------------------------------------------- decode

// One wave per expert computes the binary64 logit; the last workgroup to finish selects
// the top k with one wave (k rounds of a wave arg-max), certifies the choice against the
// binary64 error radii, and resolves uncertain experts with sequential sums.
__global__ __launch_bounds__(64) void k_decode_route(DecodeArgs a) {
  __shared__ Sel64 S;
  __shared__ int s_last;
  const int lane = threadIdx.x;
  const int e0 = blockIdx.x, H = a.H, E = a.E, k = a.k;
  {
    double l, ab;
    wave_dot64(a.x, a.wr16 ? a.wr16 + (size_t)e0 * H : nullptr, a.wr32 ? a.wr32 + (size_t)e0 * H : nullptr, H,
               lane, l, ab);
    if (a.bias) l += (double)a.bias[e0];
    if (lane == 0) {
      st_agent(&a.l64[e0], l);
      st_agent(&a.a64[e0], radius64(l, ab, H));
      vm_drain();
      s_last = ticket(&a.ctrl->decode_ticket) == E - 1;
    }
  }
  __syncthreads();
  if (!s_last) return;
  constexpr int NV = kMaxExperts / kWave;
  double v[NV], rd[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? ld_agent(&a.l64[e]) : -INFINITY;
    rd[i] = e < E ? ld_agent(&a.a64[e]) : 0.0;
    if (e < E) {
      S.gl[e] = v[i];
      S.chosen[e] = 0;
    }
  }
  uint32_t taken = 0;
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi < E && (bi % kWave) == lane) taken |= 1u << (bi / kWave);
  }
  double mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    if (e >= E) continue;
    if ((taken >> i) & 1u)
      mn = fmin(mn, v[i] - rd[i]);
    else
      mx = fmax(mx, v[i] + rd[i]);
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    mn = fmin(mn, __shfl_xor(mn, o));
    mx = fmax(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) S.n = 0;
  __syncthreads();
  int nin1 = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    if (e >= E) continue;
    const bool in_sel = (taken >> i) & 1u;
    const bool sure_in = in_sel && v[i] - rd[i] > mx;
    const bool sure_out = !in_sel && v[i] + rd[i] < mn;
    if (sure_in) {
      S.chosen[e] = 1;
      ++nin1;
    }
    if (!sure_in && !sure_out) {
      const int c = atomicAdd(&S.n, 1);
      S.cand[c] = e;
      S.v[c] = v[i];
      S.rad[c] = rd[i];
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) nin1 += __shfl_xor(nin1, o);
  __syncthreads();
  if (S.n > 0) resolve64(S, k - nin1, a.x, a.wr16, a.wr32, a.bias, H, lane, kWave);
  emit_selection(S, E, k, a.ids, a.gates, a.dbg_ids, a.dbg_gates, lane, kWave);
  if (lane == 0) st_agent(&a.ctrl->decode_ticket, 0);
}

__global__ void k_ctrl_init(Ctrl *c) {
  int *p = (int *)c;
  for (int i = threadIdx.x; i < (int)(sizeof(Ctrl) / sizeof(int)); i += blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(k_route, dim3(nb), dim3(kRouteThreads), 0, s, a);
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
