// Decode form for a batch of T = 2..8 tokens in a single launch: router logits, top-k
// selection, the gate/up GEMVs with SwiGLU and the down GEMVs with the gate-weighted
// combine.  (One token runs the kernel of decode1.hip.)
//
// "Optimizing on-device inference for Apple Silicon", section "Decode > Optimize the
// one-row weight path": a group of lanes shares one output row, each lane reading a
// different part of the packed weight row.  Section "Decode > Reduce intermediate and
// state traffic": the two input projections and the gated activation are one step; the
// output projection, the routing weights and the shared expert's result are another.
// Section "Decode > Keep every decode step on the GPU": the whole layer runs without the
// host.  Section "Limits of further optimization": verification batches of a few rows
// are an inefficient shape for one-row kernels and read experts again; here a batch of
// T <= 8 rows reads each active expert once (the union of the tokens' experts) and
// applies it to every token that chose it.
//
// Batch-1 decode moves every active weight byte once, so the layer is bound by HBM reads
// and by the latency of its dependency chain (logits -> selection -> gate/up -> down).
// One launch covers the chain.  Workgroups hand results to each other as tagged records
// (an 8-byte word holding a 32-bit value and the call's 32-bit tag, written with one
// device-scope store and read with device-scope loads, so a reader accepts a value
// exactly when its tag is this call's) or as plain device-scope stores followed by a
// tagged flag once they have completed.  The tag comes from call counters in the
// workspace, one ticket per workgroup at its start (epoch_ticket), shared with the
// one-token kernel.  The launch arguments are therefore the same for every call, so a
// sequence of calls can be captured once in a HIP graph and replayed.
//   1. the shared expert's gate/up tasks need no routing and run first;
//   2. router: every wave of the grid computes one expert's binary64 logits for a pair of
//      tokens and publishes them with their error radii (done first, before step 1's
//      tasks, since every selection waits for all of them);
//   3. workgroup t (t < T) selects token t's top k (one wave, certified against the
//      radii; the four-wave exact path when the certificate fails) and publishes the
//      chosen experts (ascending) and their softmax gates;
//   4. every workgroup with routed work reads the T selections and forms the list of
//      active experts: the shared one first, then the chosen ones in ascending order,
//      each with the set of tokens that use it;
//   5. gate/up task (active expert, 16 rows) dequantises its rows once and multiplies
//      them with every token of the expert; h goes out with device-scope stores and a
//      tagged flag per task;
//   6. down task (active expert, 64 output rows) waits for the expert's gate/up flags,
//      stages h as bf16 in LDS, and writes gate * (W_down h) per token; each (token, row
//      block) counts its k+1 arrivals and the last one sums the k+1 slots in slot order
//      (routed experts ascending, then the shared one) and writes the bf16 output.
// Every workgroup of the grid is resident at once (the grid is capped by the occupancy
// of this kernel), so each wait ends; a wait that exceeds its poll budget sets an error
// word instead of hanging.
//
// GEMV arithmetic: the dot product of a weight row with v uses the codes directly,
//     sum_k v_k (s q_k + b) = s * sum_k v_k (128 + q_k) + (b - 128 s) * sum_k v_k
// per group of 64: each 4-bit code becomes the exact bf16 number 128 + q by placing it in
// the low mantissa bits of 128 (0x4300), and v_dot2_f32_bf16 multiplies code pairs with
// bf16 activation pairs (x is bf16; h is rounded to bf16 when staged).
#include <algorithm>

#include "common.hpp"

// Every fused multiply-add below is written out, so the arithmetic of a row is the same
// in every template instance (the output of a row does not depend on the batch size).
#pragma clang fp contract(off)
#include "kernels.hpp"
#include "select64.hpp"

namespace moe {

namespace {

constexpr int kDecThreads = 256;      // four waves
constexpr int kHbWords = 8192;        // LDS words of staged h (bf16 pairs) per down round
constexpr int kSpins = 1 << 20;       // polls before a wait gives up (about a second)
constexpr int kActMax = kMaxDecodeT * kMaxTopK + 1;
constexpr int kSrecRep = 16;          // copies of the selection records

// This call's record tag (set by thread 0 at the start of k_decode).
__shared__ uint32_t s_epoch;

__device__ __forceinline__ QMat expert_mat(const QMat &routed, const QMat &shared, int e, int E, int N, int K) {
  if (e == E) return shared;
  QMat m;
  m.q = routed.q + (size_t)e * N * (K / 8);
  m.s = routed.s + (size_t)e * N * (K / 64);
  m.b = routed.b + (size_t)e * N * (K / 64);
  return m;
}

__device__ __forceinline__ uint64_t tagged(uint32_t epoch, uint32_t v) { return ((uint64_t)epoch << 32) | v; }
__device__ __forceinline__ uint32_t tag_of(uint64_t r) { return (uint32_t)(r >> 32); }

// The eight 4-bit codes of a word as four bf16 pairs holding 128 + code (exact): codes
// 2j, 2j+1 are byte j of the low and of the high nibbles.
__device__ __forceinline__ void codes_bf16(uint32_t w, uint32_t *o) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = (uint32_t)j | 0x0c00u | ((uint32_t)(4 + j) << 16) | 0x0c000000u;
    o[j] = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
  }
}

// sum over 32 elements of (128 + q) v with the codes of a 16-byte chunk converted by
// codes_bf16 (16 words) and v as 16 bf16 pairs
__device__ __forceinline__ float dot32(const uint32_t (&o)[16], const uint32_t *v) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) d = dot2_bf16(o[i], v[i], d);
  return d;
}
__device__ __forceinline__ float sum32(const uint32_t *v) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) d = dot2_bf16(0x3f803f80u, v[i], d);  // pairs of 1.0
  return d;
}

struct DecShared {
  Sel64 S;
  uint32_t cand[kDecThreads / kWave][kMaxTopK];  // each wave's top-k keys
  int wcnt[kDecThreads / kWave];
  float wf[kDecThreads / kWave];
  double red[2][4];
  int fast;                                      // the one-wave selection was certified
  int ids[kMaxDecodeT][kMaxTopK];                // every token's experts, ascending
  float gates[kMaxDecodeT][kMaxTopK];
  uint32_t emask[kMaxExperts + 1];               // tokens that chose each expert
  int act_e[kActMax];                            // active experts: shared first, then ascending
  uint32_t act_m[kActMax];                       // their token masks
  int n_act;
  int arrive[kMaxDecodeT];                       // this workgroup completed (token, row block)
  float sgz[kDecThreads / kWave][kMaxDecodeT];   // shared gate: per-wave partial dot products
  float sgv[kMaxDecodeT];                        // weight of the shared expert per token
  __attribute__((aligned(16))) uint32_t hb[kHbWords];  // staged h, bf16 pairs
};

// ------------------------------------------------------------------ router (binary64)

// Additions on any path of router_dot's sum: H/64 per lane, a 6-level butterfly.
__device__ __forceinline__ int router_depth(int H) { return H / 64 + 6; }

// Binary64 logits of expert e for tokens t0 .. t0+TT-1 (those below T), by one wave: lane
// takes the 8-element chunks c = lane + 64 i of the router row (read once) and sums the
// exact products of each token sequentially; a butterfly gives every lane the totals.
// The loads of four chunks of the row (and of the first token) are issued before any is
// used.  router_pub: lane 0 publishes (t, e)'s three records: the two halves of the
// logit (+ bias) and its error radius.
template <int TT>
__device__ void router_dot(const DecodeArgs &a, int e, int t0, double (&l)[TT], double (&ab)[TT]) {
  const int lane = threadIdx.x & 63, H = a.H, T = a.T - t0;
  const uint16_t *xb = a.x + (size_t)t0 * H;
  constexpr int B4 = 4;
  double s[TT], sa[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) s[t] = sa[t] = 0.0;
  for (int c0 = lane; c0 < H / 8; c0 += B4 * kWave) {
    uint4 w0[B4], w1[B4], xv[B4];
#pragma unroll
    for (int u = 0; u < B4; ++u) {
      const int c = c0 + u * kWave;
      const int cc = c < H / 8 ? c : lane;  // past the row: a valid chunk, skipped below
      if (a.wr16) {
        w0[u] = *(const uint4 *)(a.wr16 + (size_t)e * H + 8 * cc);
      } else {
        w0[u] = *(const uint4 *)(a.wr32 + (size_t)e * H + 8 * cc);
        w1[u] = *(const uint4 *)(a.wr32 + (size_t)e * H + 8 * cc + 4);
      }
      xv[u] = *(const uint4 *)(xb + 8 * cc);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= T) break;
      if (t > 0) {
#pragma unroll
        for (int u = 0; u < B4; ++u) {
          const int c = c0 + u * kWave;
          xv[u] = *(const uint4 *)(xb + (size_t)t * H + 8 * (c < H / 8 ? c : lane));
        }
      }
#pragma unroll
      for (int u = 0; u < B4; ++u) {
        if (c0 + u * kWave >= H / 8) break;
        float wf[8];
        if (a.wr16) {
          wf[0] = bf16_lo(w0[u].x); wf[1] = bf16_hi(w0[u].x); wf[2] = bf16_lo(w0[u].y); wf[3] = bf16_hi(w0[u].y);
          wf[4] = bf16_lo(w0[u].z); wf[5] = bf16_hi(w0[u].z); wf[6] = bf16_lo(w0[u].w); wf[7] = bf16_hi(w0[u].w);
        } else {
          wf[0] = __uint_as_float(w0[u].x); wf[1] = __uint_as_float(w0[u].y);
          wf[2] = __uint_as_float(w0[u].z); wf[3] = __uint_as_float(w0[u].w);
          wf[4] = __uint_as_float(w1[u].x); wf[5] = __uint_as_float(w1[u].y);
          wf[6] = __uint_as_float(w1[u].z); wf[7] = __uint_as_float(w1[u].w);
        }
        const float xf[8] = {bf16_lo(xv[u].x), bf16_hi(xv[u].x), bf16_lo(xv[u].y), bf16_hi(xv[u].y),
                             bf16_lo(xv[u].z), bf16_hi(xv[u].z), bf16_lo(xv[u].w), bf16_hi(xv[u].w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double p = (double)xf[i] * (double)wf[i];  // exact
          s[t] += p;
          sa[t] += fabs(p);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    l[t] = wave_sum_f64(s[t]);
    ab[t] = wave_sum_f64(sa[t]);
    if (a.bias) l[t] += (double)a.bias[e];
  }
}
template <int TT>
__device__ void router_pub(const DecodeArgs &a, int e, int t0, const double (&l)[TT], const double (&ab)[TT]) {
  const int lane = threadIdx.x & 63, H = a.H, E = a.E, T = a.T - t0;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t >= T) break;
    if (lane == 0) {
      const uint64_t lb = (uint64_t)__double_as_longlong(l[t]);
      const float rad = __double2float_ru(radius64(l[t], ab[t], H, router_depth(H)));
      uint64_t *rec = a.lrec + 3 * ((size_t)(t0 + t) * E + e);
      st_agent(&rec[0], tagged(s_epoch, (uint32_t)lb));
      st_agent(&rec[1], tagged(s_epoch, (uint32_t)(lb >> 32)));
      st_agent(&rec[2], tagged(s_epoch, __float_as_uint(rad)));
    }
  }
}

// ------------------------------------------------------------------ selection

// Wait for expert e's three logit records of token t.
__device__ void read_logit(const DecodeArgs &a, int t, int e, double &v, double &r) {
  const uint64_t *rec = a.lrec + 3 * ((size_t)t * a.E + e);
  for (int i = 0;; ++i) {
    const uint64_t r0 = ld_agent(&rec[0]), r1 = ld_agent(&rec[1]), r2 = ld_agent(&rec[2]);
    if (tag_of(r0) == s_epoch && tag_of(r1) == s_epoch && tag_of(r2) == s_epoch) {
      v = __longlong_as_double((long long)(((uint64_t)(uint32_t)r1 << 32) | (uint32_t)r0));
      r = (double)__uint_as_float((uint32_t)r2);
      return;
    }
    if (i == kSpins) {
      st_agent(&a.ctrl->d_err, 1);
      v = -INFINITY;
      r = 0.0;
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Order-preserving 32-bit key of a logit of expert e: the fp32 value's ordered bits with
// the low 8 replaced by the complemented index, so the largest key is the largest logit,
// ties (and logits equal in their top 24 bits) to the lower index.  The truncation only
// changes the choice between logits much closer than 2^-15 relative; the certificate
// below, on the binary64 values and radii, catches any such choice.
__device__ __forceinline__ uint32_t logit_key(double v, int e) {
  const uint32_t b = __float_as_uint((float)v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (ord & 0xffffff00u) | (uint32_t)(255 - e);
}

// Top-k of token t's E logits by one wave (four experts per lane): k rounds of a wave
// maximum over the keys, then the certificate (every chosen logit minus its radius above
// every other logit plus its radius).  Ids ascending and softmax gates into sh.ids[t],
// sh.gates[t].  The lane's twelve records are loaded together and re-polled together.
// Returns false, having written nothing, when the certificate fails.
__device__ bool select_topk_wave(const DecodeArgs &a, DecShared &sh, int t) {
  constexpr int NV = kMaxExperts / kWave;
  const int lane = threadIdx.x & 63, E = a.E, k = a.k;
  double v[NV], r[NV];
  bool valid[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) valid[i] = lane + kWave * i < E;
  const uint64_t *base = a.lrec + 3 * (size_t)t * E;
  uint64_t rec[NV][3];
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) rec[i][j] = valid[i] ? ld_agent(&base[3 * (size_t)(lane + kWave * i) + j]) : 0u;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) ok &= !valid[i] || tag_of(rec[i][j]) == s_epoch;
    if (__ballot(!ok) == 0ull) break;
    if (it == kSpins) {  // as read_logit: flag the error, missing logits count as -inf
      st_agent(&a.ctrl->d_err, 1);
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (valid[i] && (tag_of(rec[i][0]) != s_epoch || tag_of(rec[i][1]) != s_epoch || tag_of(rec[i][2]) != s_epoch))
          rec[i][0] = 0u, rec[i][1] = (uint64_t)0xfff00000u, rec[i][2] = 0u;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = valid[i] ? __longlong_as_double((long long)(((uint64_t)(uint32_t)rec[i][1] << 32) | (uint32_t)rec[i][0]))
                    : -INFINITY;
    r[i] = valid[i] ? (double)__uint_as_float((uint32_t)rec[i][2]) : 0.0;
    key[i] = valid[i] ? logit_key(v[i], lane + kWave * i) : 0u;
  }
  uint32_t chosen = 0;
  for (int rr = 0; rr < k; ++rr) {
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) best = max(best, key[i]);
    best = wave_max_u32(best);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (key[i] == best && best != 0u) key[i] = 0u, chosen |= 1u << i;
  }
  double mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!valid[i]) continue;
    if ((chosen >> i) & 1u)
      mn = fmin(mn, v[i] - r[i]);
    else
      mx = fmax(mx, v[i] + r[i]);
  }
  wave_minmax_f64(mn, mx);
  if (!(mn > mx)) return false;  // false for NaN or an infinite radius as well
  // softmax of the chosen logits (as fp32), ids ascending
  float gmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if ((chosen >> i) & 1u) gmax = fmaxf(gmax, (float)v[i]);
  gmax = wave_max(gmax);
  float ex[NV], part = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    ex[i] = ((chosen >> i) & 1u) ? __expf((float)v[i] - gmax) : 0.0f;
    part += ex[i];
  }
  const float den = wave_sum(part);
  int below = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool ch = (chosen >> i) & 1u;
    const uint64_t bal = __ballot(ch);
    const int pos = below + __popcll(bal & ((1ull << lane) - 1ull));
    if (ch && pos < kMaxTopK) {
      sh.ids[t][pos] = lane + kWave * i;
      sh.gates[t][pos] = ex[i] / den;
    }
    below += __popcll(bal);
  }
  return true;
}

// Top-k of token t (value descending, index ascending) into sh.ids[t] (ascending) and
// sh.gates[t]: select_topk_wave, or when its certificate fails the four-wave path below.
// One expert per thread (E <= 256): each wave takes its top k by k rounds of a wave
// maximum; a chosen candidate is one of the 4k whose rank among them is below k.  The
// choice is certified against the binary64 error radii; experts closer than their radii
// are re-ranked by resolve64.
__device__ void select_topk(const DecodeArgs &a, DecShared &sh, int t) {
  if (threadIdx.x < kWave) {
    const bool ok = select_topk_wave(a, sh, t);
    if (threadIdx.x == 0) sh.fast = ok;
  }
  __syncthreads();
  if (sh.fast) return;  // uniform
  Sel64 &S = sh.S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, E = a.E, k = a.k;
  const bool mine = tid < E;
  double v = -INFINITY, r = 0.0;
  if (mine) {
    read_logit(a, t, tid, v, r);
    S.gl[tid] = v;
  }
  uint32_t key = mine ? logit_key(v, tid) : 0u;
  const uint32_t key0 = key;
  for (int rr = 0; rr < k; ++rr) {
    const uint32_t best = wave_max_u32(key);
    key = key == best ? 0u : key;
    if (lane == 0) sh.cand[wv][rr] = best;
  }
  __syncthreads();
  {
    // rank of my key among the 4k wave candidates (keys are distinct)
    int rank = 0;
    for (int w2 = 0; w2 < kDecThreads / kWave; ++w2)
      for (int rr = 0; rr < k; ++rr) rank += sh.cand[w2][rr] > key0 ? 1 : 0;
    S.chosen[tid] = (mine && key == 0u && rank < k) ? 1 : 0;  // key cleared: one of my wave's k
  }
  __syncthreads();
  const bool sel = mine && S.chosen[tid];
  // certification: every chosen logit minus its radius above every other plus its radius
  double mn = sel ? v - r : INFINITY, mx = (mine && !sel) ? v + r : -INFINITY;
  wave_minmax_f64(mn, mx);
  if (lane == 0) {
    sh.red[0][wv] = mn;
    sh.red[1][wv] = mx;
  }
  __syncthreads();
  mn = fmin(fmin(sh.red[0][0], sh.red[0][1]), fmin(sh.red[0][2], sh.red[0][3]));
  mx = fmax(fmax(sh.red[1][0], sh.red[1][1]), fmax(sh.red[1][2], sh.red[1][3]));
  const bool sure_in = sel && v - r > mx;
  const bool sure_out = mine && !sel && v + r < mn;
  if (!__syncthreads_and(!mine || sure_in || sure_out)) {
    if (mine) S.chosen[tid] = sure_in ? 1 : 0;
    if (tid == 0) S.n = 0;
    __syncthreads();
    if (mine && !sure_in && !sure_out) {
      const int c = atomicAdd(&S.n, 1);
      S.cand[c] = tid;
      S.v[c] = v;
      S.rad[c] = r;
    }
    const int nin1 = __syncthreads_count(sure_in);
    resolve64(S, k - nin1, a.x + (size_t)t * a.H, a.wr16, a.wr32, a.bias, a.H, tid, kDecThreads);
  }
  // ids ascending (rank of each chosen expert = chosen experts below it) and softmax
  // gates of the chosen logits
  const bool ch = mine && S.chosen[tid];
  const float gl = ch ? (float)S.gl[tid] : -INFINITY;
  const uint64_t bal = __ballot(ch);
  const uint32_t gb = __float_as_uint(gl);
  const uint32_t wo = wave_max_u32((gb & 0x80000000u) ? ~gb : (gb | 0x80000000u));  // ordered bits
  if (lane == 0) {
    sh.wcnt[wv] = __popcll(bal);
    sh.wf[wv] = __uint_as_float((wo & 0x80000000u) ? (wo & 0x7fffffffu) : ~wo);
  }
  __syncthreads();
  int below = __popcll(bal & ((1ull << lane) - 1ull));
  float gmax = -INFINITY;
  for (int w2 = 0; w2 < kDecThreads / kWave; ++w2) {
    below += w2 < wv ? sh.wcnt[w2] : 0;
    gmax = fmaxf(gmax, sh.wf[w2]);
  }
  const float ex = ch ? __expf(gl - gmax) : 0.0f;
  const float ws = wave_sum(ex);
  __syncthreads();  // every thread has read sh.wf / sh.wcnt
  if (lane == 0) sh.wf[wv] = ws;
  __syncthreads();
  const float den = (sh.wf[0] + sh.wf[1]) + (sh.wf[2] + sh.wf[3]);
  if (ch && below < kMaxTopK) {
    sh.ids[t][below] = tid;
    sh.gates[t][below] = ex / den;
  }
  __syncthreads();
  if (tid < k) sh.ids[t][tid] = min(max(sh.ids[t][tid], 0), E - 1);  // keep reads in bounds even after a failed wait
  __syncthreads();
}

// Every token's selection from the selectors' records into sh.ids / sh.gates, then the
// list of active experts (shared first, then ascending) with their token masks.
__device__ void read_routing(const DecodeArgs &a, DecShared &sh, int rep) {
  const int tid = threadIdx.x, T = a.T, E = a.E, k = a.k;
  if (tid < kWave) {
    const int n = T * 2 * k;  // <= 256
    uint64_t rec[4];
    for (int it = 0;; ++it) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tid + kWave * i;
        rec[i] = j < n ? ld_agent(&a.srec[(size_t)rep * n + j]) : tagged(s_epoch, 0u);
        ok &= tag_of(rec[i]) == s_epoch;
      }
      if (__ballot(!ok) == 0ull) break;
      if (it == kSpins) {
        st_agent(&a.ctrl->d_err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = tid + kWave * i;
      if (j >= n) continue;
      const int t = j / (2 * k), q = j - t * 2 * k;
      if (q < k)
        sh.ids[t][q] = min(max((int)(uint32_t)rec[i], 0), E - 1);  // in bounds even after a failed wait
      else
        sh.gates[t][q - k] = __uint_as_float((uint32_t)rec[i]);
    }
  }
  for (int e = tid; e <= E; e += kDecThreads) sh.emask[e] = e == E ? (1u << T) - 1u : 0u;
  __syncthreads();
  if (tid < T * k) atomicOr(&sh.emask[sh.ids[tid / k][tid % k]], 1u << (tid / k));
  __syncthreads();
  if (tid < kWave) {
    int n = 1;
    if (tid == 0) {
      sh.act_e[0] = E;
      sh.act_m[0] = sh.emask[E];
    }
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + tid;
      const bool on = e < E && sh.emask[e] != 0u;
      const uint64_t bal = __ballot(on);
      if (on) {
        const int p = n + __popcll(bal & ((1ull << tid) - 1ull));
        sh.act_e[p] = e;
        sh.act_m[p] = sh.emask[e];
      }
      n += __popcll(bal);
    }
    if (tid == 0) sh.n_act = n;
  }
  __syncthreads();
}

// index of the n-th set bit of m (n < popcount(m))
__device__ __forceinline__ int nth_bit(uint32_t m, int n) {
  for (int i = 0; i < n; ++i) m &= m - 1u;
  return __ffs((int)m) - 1;
}

// slot of expert u in token t's selection (k for the shared expert)
__device__ __forceinline__ int slot_of(const DecodeArgs &a, const DecShared &sh, int t, int u) {
  if (u == a.E) return a.k;
  int j = 0;
  for (int q = 0; q < a.k; ++q) j = sh.ids[t][q] == u ? q : j;
  return j;
}

// ------------------------------------------------------------------ gate/up

// Gate/up task: rows rb*16 .. rb*16+15 of active expert `act` (expert u, tokens tm);
// wave w takes rows rb*16 + 4w .. rb*16 + 4w + 3; lane takes the 32-element chunks
// c = lane + 64 i.  The loads of all four rows of a chunk are issued before any is used;
// each row's codes are converted once and multiplied with every token.  h of (t, slot,
// row) goes out with device-scope stores; after all four waves' stores have completed,
// the task's tagged flag.
template <int TT>
__device__ void gu_task(const DecodeArgs &a, DecShared &sh, int act, int u, uint32_t tm, int rb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I, E = a.E, k = a.k;
  const QMat Gm = expert_mat(a.gate, a.s_gate, u, E, I, H), Um = expert_mat(a.up, a.s_up, u, E, I, H);
  const int r0 = rb * kDecGuTask + 4 * wv;  // rows r0 .. r0+3 (r0 a multiple of 4)
  float acc[TT][4][2];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r][0] = acc[t][r][1] = 0.f;
  for (int c = lane; c < H / 32; c += kWave) {
    uint4 cw[2][4];
    uint32_t sv[2][2], bv[2][2];  // per matrix and row pair: fp16 scale / bias of the two rows
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const QMat &M = m ? Um : Gm;
#pragma unroll
      for (int r = 0; r < 4; ++r) cw[m][r] = *(const uint4 *)(M.q + code_index((size_t)(r0 + r), 4 * c, H));
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const size_t qi = qp_index((size_t)(r0 + 2 * pp), c / 2, H / 64);
        sv[m][pp] = *(const uint32_t *)(M.s + qi);
        bv[m][pp] = *(const uint32_t *)(M.b + qi);
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      uint32_t o[2][2][16];
      float s[2][2], b2[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint4 &w = cw[m][2 * pp + r];
          codes_bf16(w.x, &o[m][r][0]);
          codes_bf16(w.y, &o[m][r][4]);
          codes_bf16(w.z, &o[m][r][8]);
          codes_bf16(w.w, &o[m][r][12]);
          s[m][r] = qp_f32(sv[m][pp] >> (16 * r), a.qbf16);
          b2[m][r] = __builtin_fmaf(-128.0f, s[m][r], qp_f32(bv[m][pp] >> (16 * r), a.qbf16));
        }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (!((tm >> t) & 1u)) continue;
        uint32_t xw[16];
        const uint4 *xp = (const uint4 *)(a.x + (size_t)t * H + 32 * c);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 xq = xp[v];
          xw[4 * v] = xq.x; xw[4 * v + 1] = xq.y; xw[4 * v + 2] = xq.z; xw[4 * v + 3] = xq.w;
        }
        const float xs = sum32(xw);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[t][2 * pp + r][m] =
                __builtin_fmaf(s[m][r], dot32(o[m][r], xw), __builtin_fmaf(b2[m][r], xs, acc[t][2 * pp + r][m]));
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (!((tm >> t) & 1u)) continue;
    const int j = slot_of(a, sh, t, u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gs = wave_sum(acc[t][r][0]);
      const float us = wave_sum(acc[t][r][1]);
      const float hv = gs / (1.0f + __expf(-gs)) * us;
      if (lane == r) st_agent(&a.hval[((size_t)t * (k + 1) + j) * I + r0 + r], hv);
    }
  }
  vm_drain();  // this wave's h stores have completed
  __syncthreads();
  if (threadIdx.x == 0) st_agent(&a.hflag[(size_t)act * (I / kDecGuTask) + rb], tagged(s_epoch, 1u));
}

// ------------------------------------------------------------------ down

// Down task: output rows n0 = rb*64 .. n0+63 of active expert `act` (expert u, tokens tm).
// Waits for the expert's I/16 gate/up flags, stages each token's h as bf16 pairs in LDS
// (in rounds when they do not fit), then 16-lane group q of wave w takes rows
// n0 + 16w + 4i + q (i < 4), lane cl = lane%16 the 32-element chunks c = cl + 16p.  Writes
// gate * y per (token, slot, row) and counts the (token, row block) arrivals; the
// workgroup that completes a (token, row block) sums its k+1 slots in slot order.
// The weights of one chunk c of a down task (the lane's four rows), in plain words (a union
// vector type kept across calls here is not split into registers).  The first chunk
// (c = lane % 16) of a workgroup's first down task is loaded before the expert's h is
// ready.
struct DnPre {
  uint32_t w[4][4];     // code words
  uint32_t s[4], b[4];  // fp16 bits
};

__device__ __forceinline__ void dn_load(const DecodeArgs &a, int u, int rb, int c, DnPre &P) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, q = lane >> 4;
  const int H = a.H, I = a.I;
  if (c >= I / 32) return;  // no such chunk for this lane (I = 128, 256, 384)
  const QMat D = expert_mat(a.down, a.s_down, u, a.E, H, I);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t n = (size_t)(rb * kDecDnTask + 16 * wv + 4 * i + q);
    const uint4 v = *(const uint4 *)(D.q + code_index(n, 4 * c, I));
    P.w[i][0] = v.x;
    P.w[i][1] = v.y;
    P.w[i][2] = v.z;
    P.w[i][3] = v.w;
    const size_t qi = qp_index(n, c / 2, I / 64);
    P.s[i] = D.s[qi];
    P.b[i] = D.b[qi];
  }
}

// Down task: output rows n0 = rb*64 .. n0+63 of active expert `act` (expert u, tokens tm).
// Waits for the expert's I/16 gate/up flags, stages each token's h as bf16 pairs in LDS
// (in rounds when they do not fit), then 16-lane group q of wave w takes rows
// n0 + 16w + 4i + q (i < 4), lane cl = lane%16 the 32-element chunks c = cl + 16p (the
// first one's weights in `pre`).  Writes gate * y per (token, slot, row) and counts the
// (token, row block) arrivals; the workgroup that completes a (token, row block) sums its
// k+1 slots in slot order.
template <int TT>
__device__ __forceinline__ void dn_task(const DecodeArgs &a, DecShared &sh, int act, int u, uint32_t tm, int rb,
                                        DnPre pre) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, q = lane >> 4, cl = lane & 15;
  const int H = a.H, I = a.I, k = a.k;
  const int ntb = I / kDecGuTask;
  // 1. the expert's gate/up tasks are done
  if (tid < kWave) {
    const uint64_t *fl = a.hflag + (size_t)act * ntb;
    for (int it = 0;; ++it) {
      bool ok = true;
      for (int i = tid; i < ntb; i += kWave) ok &= tag_of(ld_agent(&fl[i])) == s_epoch;
      if (__ballot(!ok) == 0ull) break;
      if (it == kSpins) {
        st_agent(&a.ctrl->d_err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  const int n0 = rb * kDecDnTask;
  const int nt = __popc(tm);
  const int per_round = kHbWords / (I / 2);  // tokens whose h fits in LDS at once (>= 4)
  // the shared expert's weight per token: sigmoid(x_t . w_sg), or 1
  if (u == a.E) {
    if (a.sgate) {
      float z[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) z[t] = 0.f;
      for (int c = tid; c < H / 8; c += kDecThreads) {
        const uint4 wv4 = *(const uint4 *)(a.sgate + 8 * c);
        const uint32_t ww[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          if (t >= a.T) break;
          const uint4 xv = *(const uint4 *)(a.x + (size_t)t * H + 8 * c);
          const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) z[t] = dot2_bf16(xw[i], ww[i], z[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float zs = wave_sum(z[t]);
        if (lane == 0) sh.sgz[wv][t] = zs;
      }
    }
    __syncthreads();
    if (tid < TT) {
      const float zt = (sh.sgz[0][tid] + sh.sgz[1][tid]) + (sh.sgz[2][tid] + sh.sgz[3][tid]);
      sh.sgv[tid] = a.sgate ? 1.0f / (1.0f + __expf(-zt)) : 1.0f;
    }
  }
  for (int t0 = 0; t0 < nt; t0 += per_round) {
    const int nb = min(per_round, nt - t0);
    if (t0 > 0) dn_load(a, u, rb, cl, pre);
    __syncthreads();  // the flags are seen (first round) / the previous round's reads are done
    for (int i = tid; i < nb * (I / 2); i += kDecThreads) {
      const int ti = i / (I / 2), w = i - ti * (I / 2);
      const int t = nth_bit(tm, t0 + ti);
      const float *hp = a.hval + ((size_t)t * (k + 1) + slot_of(a, sh, t, u)) * I + 2 * w;
      sh.hb[ti * (I / 2) + w] = pack_bf16x2(ld_agent(hp), ld_agent(hp + 1));
    }
    __syncthreads();
    float acc[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = 0.f;
    auto chunk = [&](int c, const DnPre &W) {
      uint32_t o[4][16];
      float s[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = qp_f32(W.s[i], a.qbf16);
        b2[i] = __builtin_fmaf(-128.0f, s[i], qp_f32(W.b[i], a.qbf16));
#pragma unroll
        for (int v = 0; v < 4; ++v) codes_bf16(W.w[i][v], &o[i][4 * v]);
      }
#pragma unroll
      for (int ti = 0; ti < TT; ++ti) {
        if (ti >= nb) break;
        const uint32_t *hp = &sh.hb[ti * (I / 2) + 16 * c];
        uint32_t hw[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 x4 = *(const uint4 *)(hp + 4 * v);
          hw[4 * v] = x4.x; hw[4 * v + 1] = x4.y; hw[4 * v + 2] = x4.z; hw[4 * v + 3] = x4.w;
        }
        const float hs = sum32(hw);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[ti][i] = __builtin_fmaf(s[i], dot32(o[i], hw), __builtin_fmaf(b2[i], hs, acc[ti][i]));
      }
    };
    if (cl < I / 32) chunk(cl, pre);
    for (int c = cl + 16; c < I / 32; c += 16) {
      DnPre L;
      dn_load(a, u, rb, c, L);
      chunk(c, L);
    }
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) {
      if (ti >= nb) break;
      const int t = nth_bit(tm, t0 + ti);
      const int j = slot_of(a, sh, t, u);
      const float g = j < k ? sh.gates[t][j] : sh.sgv[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = row16_sum(acc[ti][i]);
        const float gy = g * y;
        if (cl == 0) st_agent(&a.part[((size_t)t * (k + 1) + j) * H + n0 + 16 * wv + 4 * i + q], gy);
      }
    }
  }
  vm_drain();  // this thread's partial outputs have completed
  __syncthreads();
  if (tid < nt) {  // one thread per token: the tickets are taken together
    const int t = nth_bit(tm, tid);
    int *ctr = a.rbctr + ((size_t)t * (H / kDecDnTask) + rb) * kCtrStride;
    const int c = ticket(ctr);
    sh.arrive[tid] = c == k;  // the (k+1)-th arrival
    if (c == k) st_agent(ctr, 0);
  }
  __syncthreads();
  // the (token, row block)s this workgroup completed: sum the k+1 slots in slot order
  for (int i = 0; i < nt; ++i) {
    if (!sh.arrive[i]) continue;  // uniform
    const int t = nth_bit(tm, i);
    if (tid < kDecDnTask) {
      const float *pp = a.part + (size_t)t * (k + 1) * H + n0 + tid;
      float v[kMaxTopK + 1];
#pragma unroll
      for (int j = 0; j <= kMaxTopK; ++j) v[j] = j <= k ? ld_agent(pp + (size_t)j * H) : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j <= kMaxTopK; ++j) sum += j <= k ? v[j] : 0.f;
      a.out[(size_t)t * H + n0 + tid] = f32_to_bf16(sum);
    }
  }
}

// ------------------------------------------------------------------ the layer

// Workgroups start XCD by XCD (workgroup b on the XCD b mod 8 under the round-robin
// placement), the XCD of workgroup 0 first and the others up to a few microseconds
// later.  The router is spread over every wave of the grid (every selection waits for
// all of it); the selections go to the workgroups b = 0 mod 8; the shared expert's
// gate/up tasks, which need no routing, to b = 1 mod 8, the next XCD to start; the other
// tasks follow.  pos(b) orders the workgroups by residue 1, 2, ..., 7, 0 (then by b).
__device__ __forceinline__ int wg_pos(int b, int G) {
  const int r = b % 8, ri = (r + 7) % 8;  // residue 1 -> 0, ..., 0 -> 7
  int before = 0;
  for (int j = 0; j < ri; ++j) {
    const int rj = (j + 1) % 8;
    before += G / 8 + (rj < G % 8 ? 1 : 0);
  }
  return before + b / 8;
}

// Two waves per SIMD (two workgroups per CU, so one's memory round trips overlap the
// other's work) where the registers allow it without heavy spilling: up to four rows
// (measured 35.8 -> 33.6 us at two rows, 52.5 -> 47.6 at four); eight rows would spill
// 636 bytes per lane and ran 111 -> 132 us, so they keep one wave per SIMD.
template <int TT>
__global__ __launch_bounds__(kDecThreads, TT <= 4 ? 2 : 1) void k_decode(DecodeArgs a) {
  __shared__ DecShared sh;
  const int b = blockIdx.x, G = gridDim.x, tid = threadIdx.x, wv = tid >> 6;
  // the call's ticket goes out now; wave 0 reads it back after its router loads (so the
  // router does not wait for the atomic's round trip), then a barrier shares the tag
  uint64_t tk;
  if (tid == 0) tk = epoch_ticket(a.epctr, kCtrStride / 2, b, G);
  const int T = a.T, E = a.E, k = a.k;
  const int ntb = a.I / kDecGuTask;       // gate/up tasks per active expert
  const int nrb = a.H / kDecDnTask;       // down tasks per active expert
  const int act_max = min(T * k, E) + 1;
  const uint32_t all_tok = (1u << T) - 1u;
  const int gpos = wg_pos(b, G);          // gate/up tasks g = gpos, gpos + G, ...
  const bool spread_sel = 8 * (T - 1) < G;
  const bool selector = spread_sel ? (b % 8 == 0 && b / 8 < T) : b < T;
  const int my_tok = spread_sel ? b / 8 : b;

  // the first down task's weights, if it belongs to the shared expert (known now).  A
  // wave's loads complete in issue order, so these also hold back the router's loads and
  // the record polls behind them; with eight rows (one workgroup per CU) that costs more
  // than the early start gains, and the loads go out with the routed ones instead.
  DnPre pre;
  const bool pre_shared = TT <= 4 && b < nrb;
  if (pre_shared) dn_load(a, E, b, threadIdx.x & 15, pre);

  // 1. router logits, published as records: (expert, pair of tokens) per wave over every
  // wave of the grid, before anything else, since every selection waits for all of them
  {
    constexpr int TPW = 2;  // tokens per router wave
    const int nsub = (T + TPW - 1) / TPW, nw = 4 * G;
    int p = b * 4 + wv;
    double l[TPW], ab[TPW];
    if (p < E * nsub) router_dot<TPW>(a, p / nsub, TPW * (p % nsub), l, ab);
    if (tid < kWave) s_epoch = epoch_of(lane0_u64(tk));
    __syncthreads();  // s_epoch
    if (p < E * nsub) router_pub<TPW>(a, p / nsub, TPW * (p % nsub), l, ab);
    for (p += nw; p < E * nsub; p += nw) {
      router_dot<TPW>(a, p / nsub, TPW * (p % nsub), l, ab);
      router_pub<TPW>(a, p / nsub, TPW * (p % nsub), l, ab);
    }
  }

  // 2. the shared expert (active index 0): gate/up before the routing is known
  for (int g = gpos; g < ntb; g += G) gu_task<TT>(a, sh, 0, E, all_tok, g);

  // 3. selection of token my_tok, published as records (ids ascending, then gates), in
  // kSrecRep copies so that few workgroups poll each copy
  if (selector) {
    const int t = my_tok;
    select_topk(a, sh, t);
    for (int i = tid; i < kSrecRep * 2 * k; i += kDecThreads) {
      const int r = i / (2 * k), q = i - r * 2 * k;
      const uint32_t v = q < k ? (uint32_t)sh.ids[t][q] : __float_as_uint(sh.gates[t][q - k]);
      st_agent(&a.srec[((size_t)r * T + t) * 2 * k + q], tagged(s_epoch, v));
    }
    if (tid < k) {
      if (a.dbg_ids) a.dbg_ids[(size_t)t * k + tid] = sh.ids[t][tid];
      if (a.dbg_gates) a.dbg_gates[(size_t)t * k + tid] = sh.gates[t][tid];
    }
  }

  // 4. the routing, in every workgroup that may have routed work
  int g_next = gpos;
  while (g_next < ntb) g_next += G;
  const bool may_gu = g_next < ntb * act_max;
  const bool may_dn = b < nrb * act_max;
  if (may_gu || may_dn) {
    read_routing(a, sh, b % kSrecRep);
    const int n_act = sh.n_act;
    // the first down task's weights (a routed expert's) go out with the gate/up loads
    if (!pre_shared && b < nrb * n_act) dn_load(a, sh.act_e[b / nrb], b % nrb, threadIdx.x & 15, pre);
    // 5. routed gate/up tasks
    for (int g = g_next; g < ntb * n_act; g += G) {
      const int act = g / ntb;
      gu_task<TT>(a, sh, act, sh.act_e[act], sh.act_m[act], g - act * ntb);
    }
    // 6. down tasks
    for (int d = b; d < nrb * n_act; d += G) {
      const int act = d / nrb;
      if (d != b) dn_load(a, sh.act_e[act], d - act * nrb, threadIdx.x & 15, pre);
      dn_task<TT>(a, sh, act, sh.act_e[act], sh.act_m[act], d - act * nrb, pre);
    }
  }
}

template <int TT>
int capacity_of(int n_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode<TT>, kDecThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * n_cu;
}

}  // namespace

DecodeLayout decode_layout(int H, int E, int k, int I, int t_max) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  DecodeLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = al(o + bytes);
    return at;
  };
  const size_t T = (size_t)t_max, K1 = (size_t)k + 1;
  // the call counters first, at the same offset for every shape: a region shared by the
  // plans of different layers keeps one consistent count of calls
  L.epctr = take(8 * kCtrStride * 4);
  if (t_max <= 1) {  // the one-token kernel: logit and h records only
    L.lrec = take((size_t)kLrecRep * E * 3 * 8);
    L.hrec1 = take((size_t)kHrecRep * K1 * I / 2 * 8);
    L.total = o;
    return L;
  }
  L.lrec = take(std::max<size_t>(T, kLrecRep) * E * 3 * 8);
  L.srec = take(kSrecRep * T * 2 * k * 8);
  L.hflag = take((std::min<size_t>(T * k, E) + 1) * (I / kDecGuTask) * 8);
  L.hval = take(T * K1 * I * 4);
  L.hrec1 = take((size_t)kHrecRep * K1 * I / 2 * 8);
  L.part = take(T * K1 * H * 4);
  L.rbctr = take(T * (H / kDecDnTask) * kCtrStride * 4);
  L.total = o;
  return L;
}

int decode_capacity(int t_max, int n_cu) {
  if (t_max <= 2) return capacity_of<2>(n_cu);
  if (t_max <= 4) return capacity_of<4>(n_cu);
  return capacity_of<8>(n_cu);
}

int decode_grid(const DecodeArgs &a, int capacity) {
  const int act_max = std::min(a.T * a.k, a.E) + 1;
  int want = (a.E + 3) / 4;
  want = std::max(want, act_max * (a.I / kDecGuTask));
  want = std::max(want, act_max * (a.H / kDecDnTask));
  want = std::max(want, a.T);
  return std::min(want, capacity);
}

hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t s) {
  if (a.T <= 2)
    hipLaunchKernelGGL(k_decode<2>, dim3(grid), dim3(kDecThreads), 0, s, a);
  else if (a.T <= 4)
    hipLaunchKernelGGL(k_decode<4>, dim3(grid), dim3(kDecThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode<8>, dim3(grid), dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
