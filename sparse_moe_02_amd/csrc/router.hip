// Router: logits, top-k selection with lowest-index tie-break, softmax gates.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates three
// different workload shapes": the router scores every routed expert and keeps eight
// per token.  The selection is defined on exact logits (ties: lower index wins).
//
// Prefill, two launches.  k_route_logits tiles (64 tokens x 64 experts) over the whole
// grid so every CU works and the router rows are read from L2 only T/64 times; logits
// and the bound sum_h |x_h w_eh| come from two bf16 MFMA chains with fp32 accumulation
// (bf16 x bf16 products are exact in fp32) and go to the workspace.  k_route then takes
// 32 tokens per workgroup: a token's fp32 ranking is certified when every chosen logit
// minus its error radius exceeds every other logit plus its radius; otherwise one wave
// re-ranks it: undecided experts get binary64 logits (wave-parallel sums), and experts
// that even these cannot order are summed sequentially in ascending h in binary64, which
// reproduces the exact-product sequential sum bit for bit.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "select64.hpp"

namespace moe {

namespace {

constexpr float kU32 = 5.9604644775390625e-8f;       // 2^-24
// ---------------------------------------------------------------------------- prefill

constexpr int kRouteThreads = 512;   // 8 waves: loads and re-ranks; waves 0..3 select, four tokens each
constexpr int kSelTokens = 16;       // tokens per selection workgroup (half of a token-mask block)
static_assert(2 * kSelTokens == kRouteTokens, "two selection workgroups per token-mask block");
constexpr int kKC = 128;             // k per chunk (one LDS stage, one fresh fp32 partial sum)
constexpr int kKP = 128;             // k per fresh fp32 partial sum
constexpr int kLT = 64;              // logits tile: tokens
constexpr int kLE = 64;              // logits tile: experts
constexpr int kLThreads = 512;       // eight waves: four 32x32 tiles x {logit, |x||w|} chains
constexpr int kLStages = 4;          // chunks in LDS (three loaded ahead)
constexpr int kLStage = (kLT + kLE) * kKC * 2;  // 32 KiB: two 64-k halves of x rows, then of router rows
constexpr int kLHalf = (kLT + kLE) * 128;       // one 64-k half: 64 token rows, then 64 router rows

// 16-byte piece `c` (0..7) of staged 128-byte row r: swizzled so that the MFMA operand
// reads (16 rows, same piece) hit distinct banks
__device__ __forceinline__ int roff(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Logits and error radii of a 64-token x 64-expert tile.  For each 128-k chunk the 64
// token rows and 64 router rows go global -> LDS with direct-to-LDS loads (two 64-k
// halves of 8 rows x 128 bytes per wave and operand), kLStages-1 chunks ahead.  Wave
// w < 4 multiplies token tile w&1 with expert tile (w>>1)&1; wave w+4 does the same over
// sign-cleared operands, giving sum |x w| for the error radius (two waves per SIMD, so
// each hides the other's LDS latency).  H must be a multiple of 128.  Each chunk is two
// fresh MFMA chains (even and odd slices) added to the running fp32 total, so a product
// passes through at most kKP/16 + 15 roundings in its partial and H/kKP in the total.
__global__ __launch_bounds__(kLThreads) void k_route_logits(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t st[kLStages][kLStage];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, T = a.T;
  const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
  const int m = lane & 31, hf = lane >> 5;
  const int tile = wv & 3, tt = tile & 1, et = tile >> 1;
  const bool absw = wv >= 4;
  // wave wv loads token rows 8wv..8wv+7 and router rows 8wv..8wv+7 of the tile (one
  // instruction each); lane L -> row base + L/8, physical piece L%8 holding logical piece
  // (L%8) ^ f(row).  Rows past the end repeat the last one.
  const int lr = 8 * wv + (lane >> 3);
  const int piece = (lane & 7) ^ ((lr >> 1) & 7);
  const uint32_t xoff = (uint32_t)min(t0 + lr, T - 1) * (uint32_t)H * 2u + 16u * (uint32_t)piece;
  const uint32_t woff = (uint32_t)min(e0 + lr, E - 1) * (uint32_t)H * 2u + 16u * (uint32_t)piece;
  const int nch = H / kKC;
  // Workgroups walk the k chunks from different starting points: rows are 2*H bytes
  // apart, so workgroups in step would all address the same offset within their rows.
  // The workgroups of one token block (same XCD) keep the same start, so each chunk of
  // its rows is fetched into L2 once for all of them.
  const int rot = blockIdx.x % nch;
  auto issue = [&](int c) {
    const uint32_t base = lds_addr(&st[c % kLStages][0]) + (uint32_t)wv * 1024u;
    const uint32_t kc = (uint32_t)((c + rot) % nch);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      dma16(a.x, xoff + 256u * kc + 128u * h, base + h * kLHalf);
      dma16(a.wr16, woff + 256u * kc + 128u * h, base + h * kLHalf + (uint32_t)(kLT * 128));
    }
  };
  f32x16 tot = {};
  for (int c = 0; c < kLStages - 1 && c < nch; ++c) issue(c);
  // one chunk: wait for its loads, publish them, issue the loads of chunk c+kLStages-1,
  // read all four slices' fragments
  auto stage_in = [&](int c, u32x4 (&av)[kKC / 16], u32x4 (&bv)[kKC / 16]) {
    // chunk c is complete once only the loads of chunks c+1 .. (last issued) remain
    vm_wait_dyn(4 * (min(c + kLStages - 2, nch - 1) - c));
    __syncthreads();  // chunk c visible to every wave; chunk c-1's stage is free
    if (c + kLStages - 1 < nch) issue(c + kLStages - 1);
#pragma unroll
    for (int j = 0; j < kKC / 16; ++j) {
      const uint8_t *xs = &st[c % kLStages][0] + (j >> 2) * kLHalf;
      const uint8_t *ws = xs + kLT * 128;
      av[j] = *(const u32x4 *)(xs + roff(32 * tt + m, 2 * (j & 3) + hf));
      bv[j] = *(const u32x4 *)(ws + roff(32 * et + m, 2 * (j & 3) + hf));
    }
  };
  // the same loop for both kinds of wave, the |.| waves clearing the sign bits first;
  // each chunk (128 k) is two fresh MFMA chains (even and odd slices) added to the
  // running total
  auto run = [&](auto abs_tag) {
    constexpr bool kAbs = decltype(abs_tag)::value;
    const u32x4 msk = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
    auto op = [&](const u32x4 &v) { return __builtin_bit_cast(bf16x8, kAbs ? (u32x4)(v & msk) : v); };
    for (int c = 0; c < nch; ++c) {
      u32x4 av[kKC / 16], bv[kKC / 16];
      stage_in(c, av, bv);
      f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(av[0]), op(bv[0]), (f32x16){}, 0, 0, 0);
      f32x16 acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(av[1]), op(bv[1]), (f32x16){}, 0, 0, 0);
#pragma unroll
      for (int j = 2; j < kKC / 16; ++j) {
        f32x16 &ac = (j & 1) ? acc1 : acc;
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(av[j]), op(bv[j]), ac, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) tot[j] += acc[j] + acc1[j];
    }
  };
  if (absw)
    run(std::true_type{});
  else
    run(std::false_type{});
  // the abs waves hand sum |x w| to the logit waves through LDS
  __syncthreads();
  float *ab = (float *)&st[0][0] + tile * (64 * 16);
  if (absw) {
#pragma unroll
    for (int j = 0; j < 16; ++j) ab[j * 64 + lane] = tot[j];
  }
  __syncthreads();
  if (absw) return;
  // Error radius of the fp32 logit: a product passes through at most kKP/16 + 15
  // roundings in its partial's MFMA chain and H/kKP in the running total; doubled for
  // margin, plus the bias addition, the sequential binary64 reference's own error and
  // product underflow.
  const float c32 = 2.0f * (float)(kKP / 16 + 15 + H / kKP) + 4.0f;
  const int e = e0 + 32 * et + m;
  if (e < E) {
    const float bb = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = t0 + 32 * tt + 8 * (j >> 2) + 4 * hf + (j & 3);
      if (t < T) {
        const float l = tot[j] + bb;
        const float sab = ab[j * 64 + lane];
        a.lg[(size_t)t * E + e] = l;
        a.rd[(size_t)t * E + e] = c32 * kU32 * sab * 1.01f + 2.0f * kU32 * fabsf(l) + 1e-12f * sab + 1e-30f;
      }
    }
  }
}

struct RouteSmem {
  float l[kSelTokens][kMaxExperts];  // fp32 logit (+bias)
  float r[kSelTokens][kMaxExperts];  // its error radius
  WaveSel ws[kRouteThreads / kWave];
};

// One workgroup per 16 tokens (every CU busy at 4096 tokens; the selection at one wave
// per SIMD).
//  1. fp32 logits and radii of its tokens from the workspace (or, for a float32 router,
//     none: every expert is re-ranked in binary64).
//  2. fp32 selection, sixteen lanes per token, certified against the radii.
//  3. tokens the certificate does not settle are re-ranked by one wave each, in parallel.
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) RouteSmem sm;
  __shared__ int s_sel[kSelTokens][kMaxTopK];      // chosen experts
  __shared__ float s_min_in[kSelTokens], s_max_out[kSelTokens];
  __shared__ int s_list[kSelTokens];
  __shared__ int s_nflag;
  __shared__ uint32_t s_mask[kMaxExperts];
  auto &s_l = sm.l;
  auto &s_r = sm.r;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, k = a.k;
  const int t0 = blockIdx.x * kSelTokens;
  const int nt = min(kSelTokens, a.T - t0);

  for (int e = tid; e < kMaxExperts; e += kRouteThreads) s_mask[e] = 0;
  if (tid == 0) s_nflag = 0;

  if (a.wr16 && E % 4 == 0) {
    // 16-byte loads: four of each array in flight per thread (one batch for E = 256)
    constexpr int kB = 4;
    const int E4 = E / 4;
    for (int i0 = tid; i0 < kSelTokens * E4; i0 += kRouteThreads * kB) {
      float4 lv[kB], rv[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = min(i0 + u * kRouteThreads, kSelTokens * E4 - 1);
        const int m = i / E4, e4 = i - m * E4;
        const size_t o = (size_t)(t0 + min(m, nt - 1)) * E + 4 * e4;
        lv[u] = *(const float4 *)(a.lg + o);
        rv[u] = *(const float4 *)(a.rd + o);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = i0 + u * kRouteThreads;
        if (i < kSelTokens * E4) {
          const int m = i / E4, e4 = i - m * E4;
          *(float4 *)&s_l[m][4 * e4] = lv[u];
          *(float4 *)&s_r[m][4 * e4] = rv[u];
        }
      }
    }
  } else if (a.wr16) {
    // sixteen loads of each array in flight per thread (one batch for E = 256)
    constexpr int kB = 16;
    for (int i0 = tid; i0 < kSelTokens * E; i0 += kRouteThreads * kB) {
      float lv[kB], rv[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = min(i0 + u * kRouteThreads, kSelTokens * E - 1);
        const int m = i / E, e = i - m * E;
        const size_t o = (size_t)(t0 + min(m, nt - 1)) * E + e;
        lv[u] = a.lg[o];
        rv[u] = a.rd[o];
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = i0 + u * kRouteThreads;
        if (i < kSelTokens * E) {
          const int m = i / E, e = i - m * E;
          s_l[m][e] = lv[u];
          s_r[m][e] = rv[u];
        }
      }
    }
  } else {
    for (int i = tid; i < kSelTokens * kMaxExperts; i += kRouteThreads) {
      (&s_l[0][0])[i] = 0.0f;
      (&s_r[0][0])[i] = INFINITY;
    }
  }
  __syncthreads();

  // fp32 selection: wave wv takes tokens 2wv and 2wv+1, 32 lanes (two DPP rows) per token,
  // lane q holding experts q, q+32, ...  Each (logit, expert) pair is one 32-bit key: the
  // order-preserving bits of the logit with the low 8 replaced by the complemented index,
  // so the largest key is the largest logit, ties (and logits equal in their top 24 bits)
  // to the lower index; k rounds of a 32-lane maximum pick the top k, clearing each
  // winner.  Truncating the keys only changes the choice between logits closer than their
  // error radii, and such a token fails the certificate below, which uses the exact fp32
  // values.  A 32-lane reduction is four DPP steps within each row, then the two rows of
  // the half-wave exchanged with v_permlane16_swap.
  {
    const int g = lane >> 5, q = lane & 31;
    const int m = wv * 2 + g;
    constexpr int NV = kMaxExperts / 32;
    uint32_t key[NV];
    float lv[NV], rv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 32 * i;
      lv[i] = e < E ? s_l[m][e] : -INFINITY;
      rv[i] = e < E ? s_r[m][e] : 0.0f;
      const uint32_t b = __float_as_uint(lv[i]);
      const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
      key[i] = e < E ? ((ord & 0xffffff00u) | (uint32_t)(255 - e)) : 0u;
    }
    auto half_max_u32 = [](uint32_t v) {
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
      v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
      const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return max((uint32_t)sw[0], (uint32_t)sw[1]);
    };
    auto half_max_f = [](float v) {
      v = row16_max(v);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return fmaxf(__uint_as_float((uint32_t)sw[0]), __uint_as_float((uint32_t)sw[1]));
    };
    auto half_sum_f = [](float v) {
      v = row16_sum(v);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return __uint_as_float((uint32_t)sw[0]) + __uint_as_float((uint32_t)sw[1]);
    };
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
      uint32_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) best = max(best, key[i]);
      best = half_max_u32(best);
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] = key[i] == best ? 0u : key[i];
      if (q == r) my_e = 255 - (int)(best & 0xffu);
    }
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) taken |= (key[i] == 0u && q + 32 * i < E) ? (1u << i) : 0u;
    const float my_l = q < k ? s_l[m][my_e] : -INFINITY;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = q + 32 * i;
      const bool in = (taken >> i) & 1u;
      mn = (e < E && in) ? fminf(mn, lv[i] - rv[i]) : mn;
      mx = (e < E && !in) ? fmaxf(mx, lv[i] + rv[i]) : mx;
    }
    mn = -half_max_f(-mn);
    mx = half_max_f(mx);
    const bool cert = mn > mx;  // false for NaN or an infinite radius
    if (q < k) s_sel[m][q] = my_e;
    if (q == 0) {
      s_min_in[m] = mn;
      s_max_out[m] = mx;
    }
    if (m < nt && (cert || (a.no_fallback && a.wr16))) {
      // gates: softmax of the chosen logits (lane q < k holds choice q; choice 0 is the
      // largest); ids in ascending order
      const float t0l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
      const float t1l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 32));
      const float top = g ? t1l : t0l;
      const float ex = q < k ? __expf(my_l - top) : 0.0f;
      const float den = half_sum_f(ex);
      int pos = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const int e0 = __builtin_amdgcn_readlane(my_e, j), e1 = __builtin_amdgcn_readlane(my_e, 32 + j);
        const int ej = g ? e1 : e0;
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
    WaveSel &W = sm.ws[wv];
    for (int f = wv; f < nflag; f += kRouteThreads / kWave) {
      const int m = s_list[f];
      const float lo = s_min_in[m], hi = s_max_out[m];
      const bool fp32_ok = a.wr16 != nullptr;
      // classify this lane's experts e = lane + 64 i up front (all LDS reads issued
      // together): bit i of kin / kout
      int sel[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) sel[j] = j < k ? s_sel[m][j] : -1;
      float lv[kMaxExperts / kWave], rv[kMaxExperts / kWave];
#pragma unroll
      for (int i = 0; i < kMaxExperts / kWave; ++i) {
        const int e = lane + kWave * i;
        lv[i] = e < E ? s_l[m][e] : 0.0f;
        rv[i] = e < E ? s_r[m][e] : 0.0f;
      }
      uint32_t kin = 0, kout = 0;
#pragma unroll
      for (int i = 0; i < kMaxExperts / kWave; ++i) {
        const int e = lane + kWave * i;
        bool chosen = false;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) chosen |= sel[j] == e;
        kin |= (fp32_ok && chosen && lv[i] - rv[i] > hi) ? (1u << i) : 0u;
        kout |= (fp32_ok && !chosen && lv[i] + rv[i] < lo) ? (1u << i) : 0u;
      }
      auto known_in = [&](int e) { return ((kin >> (e / kWave)) & 1u) != 0u; };
      auto known_out = [&](int e) { return ((kout >> (e / kWave)) & 1u) != 0u; };
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
  // this workgroup's 16 bits of each expert's word in the 32-token mask block (the
  // low half for even workgroups); the last workgroup of an odd count also clears the
  // high half, which no workgroup owns
  {
    uint16_t *tm = (uint16_t *)a.tokmask + (size_t)(blockIdx.x >> 1) * kMaxExperts * 2;
    const int h = blockIdx.x & 1;
    const bool clear_hi = h == 0 && blockIdx.x == gridDim.x - 1;
    for (int e = tid; e < kMaxExperts; e += kRouteThreads) {
      tm[2 * e + h] = e < E ? (uint16_t)s_mask[e] : (uint16_t)0;
      if (clear_hi) tm[2 * e + 1] = 0;
    }
  }
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
  if (a.wr16) {
    hipLaunchKernelGGL(k_route_logits, dim3((a.T + kLT - 1) / kLT, (a.E + kLE - 1) / kLE), dim3(kLThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nb = (a.T + kSelTokens - 1) / kSelTokens;
  hipLaunchKernelGGL(k_route, dim3(nb), dim3(kRouteThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ctrl_init(Ctrl *c, void *clear, size_t clear_bytes, hipStream_t s) {
  const int n = (int)(clear_bytes / 4);
  hipLaunchKernelGGL(k_ctrl_init, dim3(n > 0 ? (n + 255) / 256 : 1), dim3(256), 0, s, c, (uint32_t *)clear, n);
  return hipGetLastError();
}

}  // namespace moe
