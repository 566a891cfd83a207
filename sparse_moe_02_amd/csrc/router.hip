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
#include "common.hpp"
#include "kernels.hpp"
#include "select64.hpp"

namespace moe {

namespace {

constexpr float kU32 = 5.9604644775390625e-8f;       // 2^-24
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
        S.rad[c] = radius64(l, ab, H, wave_dot64_depth(H));
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

__global__ void k_ctrl_init(Ctrl *c, uint32_t *clear, int n_words) {
  int *p = (int *)c;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < (int)(sizeof(Ctrl) / sizeof(int)); i += blockDim.x) p[i] = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += gridDim.x * blockDim.x) clear[i] = 0;
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(k_route, dim3(nb), dim3(kRouteThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ctrl_init(Ctrl *c, void *clear, size_t clear_bytes, hipStream_t s) {
  const int n = (int)(clear_bytes / 4);
  hipLaunchKernelGGL(k_ctrl_init, dim3(n > 0 ? (n + 255) / 256 : 1), dim3(256), 0, s, c, (uint32_t *)clear, n);
  return hipGetLastError();
}

}  // namespace moe
