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
#include <type_traits>

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
constexpr int kWStages = 3;          // router-row chunks in LDS (two loaded ahead: they hit L2)
constexpr int kXStages = 12;         // token-row chunks in LDS (eleven ahead: they come from HBM)
constexpr int kXStage = kRouteTokens * kKC * 2;           // 4 KiB: 32 token rows
constexpr int kWStage = kMaxExperts * kKC * 2;            // 32 KiB: 256 router rows

// 16-byte piece `c` (0..7) of staged 128-byte row r: swizzled so that the MFMA operand
// reads (16 rows, same piece) hit distinct banks
__device__ __forceinline__ int roff(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

struct RouteSmem {
  union {
    struct {                          // logits phase
      uint8_t w[kWStages][kWStage];
      uint8_t x[kXStages][kXStage];
    } st;
    struct {                          // selection and re-ranking phase
      float l[kRouteTokens][kMaxExperts];  // fp32 logit (+bias)
      float r[kRouteTokens][kMaxExperts];  // its error radius
      WaveSel ws[kRouteThreads / kWave];
    } sel;
  };
};

// One workgroup per 32 tokens.
//  1. logits: for each 64-k chunk, the 32 token rows and all router rows go global ->
//     LDS with direct-to-LDS loads (8 rows x 128 bytes per instruction); token rows are
//     loaded eleven chunks ahead, router rows (shared by every workgroup, so L2 hits)
//     two ahead; wave w multiplies its 32 experts with the 32 tokens.  Each 128-k partial is
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
    auto issue_x = [&](int c) {
      if (wv < 4) dma16(a.x, xoff0 + 128u * (uint32_t)c, lds_addr(&sm.st.x[c % kXStages][0]) + (uint32_t)wv * 1024u);
    };
    auto issue_w = [&](int c) {
      const uint32_t base = lds_addr(&sm.st.w[c % kWStages][0]);
#pragma unroll
      for (int u = 0; u < 4; ++u) dma16(a.wr16, woff0[u] + 128u * (uint32_t)c, base + (uint32_t)(4 * wv + u) * 1024u);
    };
    const int nch = H / kKC;
    f32x16 tot = {}, acc = {}, aab = {};
    const u32x4 msk = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
    f32x16 acc1 = {}, aab1 = {};
    auto compute = [&](int c) {
      const uint8_t *xs = &sm.st.x[c % kXStages][0];
      const uint8_t *ws = &sm.st.w[c % kWStages][0];
      if ((c & 1) == 0) {
        acc = (f32x16){};
        acc1 = (f32x16){};
      }
      // all four slices' fragments first, then two independent chains per quantity
      u32x4 av[kKC / 16], bv[kKC / 16];
#pragma unroll
      for (int j = 0; j < kKC / 16; ++j) {
        av[j] = *(const u32x4 *)(xs + roff(m, 2 * j + hf));
        bv[j] = *(const u32x4 *)(ws + roff(32 * wv + m, 2 * j + hf));
      }
#pragma unroll
      for (int j = 0; j < kKC / 16; ++j) {
        f32x16 &ac = (j & 1) ? acc1 : acc;
        f32x16 &ab = (j & 1) ? aab1 : aab;
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]), __builtin_bit_cast(bf16x8, bv[j]),
                                                     ac, 0, 0, 0);
        ab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, (u32x4)(av[j] & msk)),
                                                     __builtin_bit_cast(bf16x8, (u32x4)(bv[j] & msk)), ab, 0, 0, 0);
      }
      if (c & 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) tot[j] += acc[j] + acc1[j];
      }
    };
    // prologue: token rows of chunks 0..kXStages-2, router rows of chunks 0..kWStages-2.
    // Step c issues the token rows of chunk c+kXStages-1 and then the router rows of
    // chunk c+kWStages-1; chunk c's loads are complete once only the loads issued at
    // step c-1 and later remain.
    for (int c = 0; c < kXStages - 1 && c < nch; ++c) issue_x(c);
    for (int c = 0; c < kWStages - 1 && c < nch; ++c) issue_w(c);
    int last_step = 0;  // loads issued by the previous step
    for (int c = 0; c < nch; ++c) {
      vm_wait_dyn(c == 0 ? 0 : last_step);
      __syncthreads();  // chunk c visible to every wave; chunk c-1's stages are free
      last_step = 0;
      if (c + kXStages - 1 < nch) {
        issue_x(c + kXStages - 1);
        last_step += wv < 4 ? 1 : 0;
      }
      if (c + kWStages - 1 < nch) {
        issue_w(c + kWStages - 1);
        last_step += 4;
      }
      if (active) compute(c);
    }
    __syncthreads();  // every wave is past its last stage read before the logits reuse it
    if (active) {
      // Error radius of the fp32 logit: a product passes through at most kKP/16 + 15
      // roundings in its partial's MFMA chain and H/kKP in the running total; doubled
      // for margin, plus the bias addition, the sequential binary64 reference's own
      // error and product underflow.
      const float c32 = 2.0f * (float)(kKP / 16 + 15 + H / kKP) + 4.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) aab[j] += aab1[j];
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

  // fp32 selection: wave wv takes tokens 4wv..4wv+3, sixteen lanes (one DPP row) per
  // token, lane q holding experts q, q+16, ...  Each (logit, expert) pair is one 32-bit
  // key: the order-preserving bits of the logit with the low 8 replaced by the
  // complemented index, so the largest key is the largest logit, ties (and logits equal
  // in their top 24 bits) to the lower index; k rounds of a row maximum pick the top k,
  // clearing each winner.  Truncating the keys only changes the choice between logits
  // closer than their error radii, and such a token fails the certificate below, which
  // uses the exact fp32 values.
  {
    const int g = lane >> 4, q = lane & 15;
    const int m = wv * 4 + g;
    constexpr int NV = kMaxExperts / 16;
    uint32_t key[NV];
    float lv[NV], rv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 16 * i;
      lv[i] = e < E ? s_l[m][e] : -INFINITY;
      rv[i] = e < E ? s_r[m][e] : 0.0f;
      const uint32_t b = __float_as_uint(lv[i]);
      const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
      key[i] = e < E ? ((ord & 0xffffff00u) | (uint32_t)(255 - e)) : 0u;
    }
    auto row_max_u32 = [](uint32_t v) {
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
      return v;
    };
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
      uint32_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) best = max(best, key[i]);
      best = row_max_u32(best);
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] = key[i] == best ? 0u : key[i];
      if (q == r) my_e = 255 - (int)(best & 0xffu);
    }
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) taken |= (key[i] == 0u && q + 16 * i < E) ? (1u << i) : 0u;
    const float my_l = q < k ? s_l[m][my_e] : -INFINITY;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 16 * i;
      const bool in = (taken >> i) & 1u;
      mn = (e < E && in) ? fminf(mn, lv[i] - rv[i]) : mn;
      mx = (e < E && !in) ? fmaxf(mx, lv[i] + rv[i]) : mx;
    }
    mn = -row16_max(-mn);
    mx = row16_max(mx);
    const bool cert = mn > mx;  // false for NaN or an infinite radius
    if (q < k) s_sel[m][q] = my_e;
    if (q == 0) {
      s_min_in[m] = mn;
      s_max_out[m] = mx;
    }
    if (m < nt && cert) {
      // gates: softmax of the chosen logits (lane q < k holds choice q; choice 0 is the
      // largest); ids in ascending order
      const float top = __shfl(my_l, lane & ~15);
      const float ex = q < k ? __expf(my_l - top) : 0.0f;
      const float den = row16_sum(ex);
      int pos = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const int ej = __shfl(my_e, (lane & ~15) + j);
        pos += (j < k && ej < my_e) ? 1 : 0;
      }
      if (q < k) {
        const size_t o = (size_t)(t0 + m) * k + pos;
        const float gt = ex / den;
        a.ids[o] = my_e;
        a.gates[o] = gt;
        if (a.dbg_ids) a.dbg_ids[o] = my_e;
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
