// Router: logits, top-k selection with lowest-index tie-break, softmax gates.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates three
// different workload shapes": the router scores every routed expert and keeps eight
// per token.  The selection is defined on exact logits (ties: lower index wins).
//
// Prefill: one workgroup per 32 tokens.  Logits and the bound sum_h |x_h w_eh| come
// from two bf16 MFMA chains with fp32 accumulation (bf16 x bf16 products are exact in
// fp32).  A token's fp32 ranking is certified when every chosen logit minus its error
// radius exceeds every other logit plus its radius; otherwise one wave re-ranks it:
// undecided experts get binary64 logits (wave-parallel sums), and experts that even these
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
constexpr int kKC = 64;              // k per chunk (one LDS stage)
constexpr int kKP = 128;             // k per fresh fp32 partial sum (two chunks)
constexpr int kRStages = 4;          // chunks in flight
constexpr int kXStage = kRouteTokens * kKC * 2;           // 4 KiB: 32 token rows
constexpr int kWStage = kMaxExperts * kKC * 2;            // 32 KiB: 256 router rows
constexpr int kStage = kXStage + kWStage;

// 16-byte piece `c` (0..7) of staged 128-byte row r: swizzled so that the MFMA operand
// reads (16 rows, same piece) hit distinct banks
__device__ __forceinline__ int roff(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

struct RouteSmem {
  union {
    uint8_t stage[kRStages][kStage];  // logits phase
    struct {                          // selection and re-ranking phase
      float l[kRouteTokens][kMaxExperts];  // fp32 logit (+bias)
      float r[kRouteTokens][kMaxExperts];  // its error radius
      WaveSel ws[kRouteThreads / kWave];
    } sel;
  };
};

// One workgroup per 32 tokens.
//  1. logits: for each 64-k chunk, the 32 token rows and all router rows go global ->
//     LDS with direct-to-LDS loads (8 rows x 128 bytes per instruction), four chunks in
//     flight; wave w multiplies its 32 experts with the 32 tokens.  Each 128-k partial is
//     a fresh MFMA chain added to the running fp32 total, so a product passes through at
//     most kKP/16 + 15 roundings in its partial and H/kKP in the total.  A second MFMA
//     chain over sign-cleared operands gives sum |x w| for the error radius.
//  2. fp32 selection, sixteen lanes per token, certified against the radii.
//  3. tokens the certificate does not settle are re-ranked by one wave each, in parallel.
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) RouteSmem sm;
  __shared__ int s_sel[kRouteTokens][kMaxTopK];      // chosen experts
  __shared__ float s_min_in[kRouteTokens], s_max_out[kRouteTokens];
  __shared__ int s_list[kRouteTokens];
  __shared__ int s_nflag;
  __shared__ uint32_t s_mask[kMaxExperts];
  auto &s_l = sm.sel.l;
  auto &s_r = sm.sel.r;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, k = a.k;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);

  for (int e = tid; e < kMaxExperts; e += kRouteThreads) s_mask[e] = 0;
  if (tid == 0) s_nflag = 0;

  if (a.wr16) {
    const int m = lane & 31, hf = lane >> 5;
    const int nct = (E + 31) / 32;
    const bool active = wv < nct;
    // loads of one chunk: waves 0..3 each bring 8 token rows, every wave brings its own
    // 32 router rows (4 instructions of 8 rows); lane L -> row base + L/8, physical piece
    // L%8 holding logical piece (L%8) ^ f(row)
    const int xr = 8 * wv + (lane >> 3);
    const uint32_t xoff0 =
        (uint32_t)(t0 + min(xr, nt - 1)) * (uint32_t)H * 2u + 16u * (uint32_t)((lane & 7) ^ ((xr >> 1) & 7));
    uint32_t woff0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 32 * wv + 8 * u + (lane >> 3);
      woff0[u] = (uint32_t)min(e, E - 1) * (uint32_t)H * 2u + 16u * (uint32_t)((lane & 7) ^ ((e >> 1) & 7));
    }
    const int per_chunk = 4 + (wv < 4 ? 1 : 0);
    auto issue = [&](int c, int st) {
      const uint32_t base = lds_addr(&sm.stage[st][0]);
      if (wv < 4) dma16(a.x, xoff0 + 128u * (uint32_t)c, base + (uint32_t)wv * 1024u);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dma16(a.wr16, woff0[u] + 128u * (uint32_t)c, base + (uint32_t)kXStage + (uint32_t)(4 * wv + u) * 1024u);
    };
    const int nch = H / kKC;
    f32x16 tot = {}, acc = {}, aab = {};
    const u32x4 msk = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
    auto compute = [&](int c, int st) {
      const uint8_t *xs = &sm.stage[st][0];
      const uint8_t *ws = xs + kXStage;
      if ((c & 1) == 0) acc = (f32x16){};
#pragma unroll
      for (int j = 0; j < kKC / 16; ++j) {
        const u32x4 av = *(const u32x4 *)(xs + roff(m, 2 * j + hf));
        const u32x4 bv = *(const u32x4 *)(ws + roff(32 * wv + m, 2 * j + hf));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
        aab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, (u32x4)(av & msk)),
                                                      __builtin_bit_cast(bf16x8, (u32x4)(bv & msk)), aab, 0, 0, 0);
      }
      if (c & 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) tot[j] += acc[j];
      }
    };
    // prologue: chunks 0..kRStages-2 in flight
    for (int c = 0; c < kRStages - 1 && c < nch; ++c) issue(c, c);
    for (int c = 0; c < nch; ++c) {
      const int st = c % kRStages;
      // chunk c's loads are complete once only the later chunks' loads remain
      vm_wait_dyn(per_chunk * min(kRStages - 2, nch - 1 - c));
      __syncthreads();  // chunk c visible to every wave; chunk c-1's stage is free
      if (c + kRStages - 1 < nch) issue(c + kRStages - 1, (c + kRStages - 1) % kRStages);
      if (active) compute(c, st);
    }
    __syncthreads();  // every wave is past its last stage read before the logits reuse it
    if (active) {
      // Error radius of the fp32 logit: a product passes through at most kKP/16 + 15
      // roundings in its partial's MFMA chain and H/kKP in the running total; doubled
      // for margin, plus the bias addition, the sequential binary64 reference's own
      // error and product underflow.
      const float c32 = 2.0f * (float)(kKP / 16 + 15 + H / kKP) + 4.0f;
      const int e = wv * 32 + m;
      if (e < E) {
        const float bb = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = 8 * (j >> 2) + 4 * hf + (j & 3);
          const float l = tot[j] + bb;
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
      s_list[atomicAdd(&s_nflag, 1)] = m;
    }
  }
  __syncthreads();

  // Re-ranking of the tokens the fp32 certificate did not settle, one wave per token.
  // With S~ the fp32 top-k, lo = min over S~ of (l - r) and hi = max outside of (l + r):
  // a chosen expert with l - r > hi is in for sure, an outside one with l + r < lo is
  // out for sure; the rest are candidates for rerank_wave.
  const int nflag = s_nflag;
  if (nflag) {
    WaveSel &W = sm.sel.ws[wv];
    for (int f = wv; f < nflag; f += kRouteThreads / kWave) {
      const int m = s_list[f];
      const float lo = s_min_in[m], hi = s_max_out[m];
      const bool fp32_ok = a.wr16 != nullptr;
      auto in_sel = [&](int e) {
        bool r = false;
        for (int j = 0; j < k; ++j) r |= s_sel[m][j] == e;
        return r;
      };
      auto known_in = [&](int e) { return fp32_ok && in_sel(e) && s_l[m][e] - s_r[m][e] > hi; };
      auto known_out = [&](int e) { return fp32_ok && !in_sel(e) && s_l[m][e] + s_r[m][e] < lo; };
      auto l32 = [&](int e) { return s_l[m][e]; };
      const size_t o = (size_t)(t0 + m) * k;
      rerank_wave(W, known_in, known_out, l32, E, k, a.x + (size_t)(t0 + m) * H, a.wr16, a.wr32, a.bias, H, lane,
                  a.ids + o, a.gates + o, a.dbg_ids ? a.dbg_ids + o : nullptr,
                  a.dbg_gates ? a.dbg_gates + o : nullptr);
      if (lane < k) s_sel[m][lane] = W.in_ids[lane];
      wave_sync();
    }
  }
  __syncthreads();

  // per-expert bit masks of this workgroup's tokens (histogram / rank source)
  for (int i = tid; i < nt * k; i += kRouteThreads) {
    const int m = i / k, r = i - m * k;
    atomicOr(&s_mask[s_sel[m][r]], 1u << m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) a.tokmask[(size_t)blockIdx.x * E + e] = s_mask[e];
  if (tid == 0 && nflag) atomicAdd(&a.ctrl->n_refined, nflag);
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
