// Decode form for one token in a single launch: router logits, top-k selection, the
// gate/up GEMVs with SwiGLU and the down GEMVs with the gate-weighted combine.  (Batches
// of 2..8 tokens run the union-of-experts kernel in decode.hip.)
//
// "Optimizing on-device inference for Apple Silicon", section "Decode > Optimize the
// one-row weight path": a group of lanes shares one output row, each lane reading a
// different part of the packed weight row.  Section "Decode > Reduce intermediate and
// state traffic": the two input projections and the gated activation are one step; the
// output projection, the routing weights and the shared expert's result are another.
// Section "Decode > Keep every decode step on the GPU": the token's whole layer runs
// without the host.
//
// Batch-1 decode moves every active weight byte once, so the layer is bound by HBM reads
// and by the latency of its dependency chain (logits -> selection -> gate/up -> down).
// One launch covers the chain.  Workgroups hand results to each other as tagged
// records: an 8-byte word holding a 32-bit value and the call's 32-bit epoch, written
// with one device-scope store and read with device-scope loads, so a reader accepts a
// value exactly when its tag is this call's epoch; no wait uses a counter or an atomic
// read-modify-write (those serialise on one address).  The epoch comes from call
// counters in the workspace, one ticket per workgroup at its start (epoch_ticket), so
// nothing is left to do once a workgroup's last output is stored.  The launch arguments
// are therefore the same for every call, so a sequence of calls can be captured once in
// a HIP graph and replayed.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "select64.hpp"

namespace moe {

namespace {

constexpr int kDecThreads = 256;        // four waves
constexpr int kGuRows = 4;              // gate/up rows per wave in one task
constexpr int kGuTask = 4 * kGuRows;    // rows of one gate/up task
static_assert(kGuRows == 4 && kGuTask % 4 == 0 && kQpRows % 4 == 0, "a wave reads its rows' scale/bias of one group as one 8-byte run");
constexpr int kDnRows = 8;              // output rows of one down task
constexpr int kDnUnits = 5;             // (row, slot) units per 16-lane group per round
constexpr int kDnSlots = 10;            // slots per down round: 8 rows x 10 = 16 groups x 5
constexpr int kHStage = 5120;           // h values staged in LDS per down round
// In LDS every 32-element chunk of staged h (16 words of bf16 pairs) takes 20 words: the
// 16 lanes of a group read chunks c = lane%16 with 16-byte loads, and an 80-byte chunk
// stride puts them on 16 different groups of 4 banks (a 64-byte stride would put four
// lanes on each).
constexpr int kHChunkWords = 20;
constexpr int kSpins = 1 << 20;         // polls before a wait gives up (about a second)

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

// GEMV arithmetic: per group of 64, sum_i v_i (s q_i + b) = s sum_i v_i (128 + q_i) +
// (b - 128 s) sum_i v_i, with 128 + q exact in bf16 (code_pair) and v_dot2_f32_bf16 taking
// two products per instruction.  dot_chunk: sum over the 32 elements of a chunk of
// (128 + code) v, the codes of four packed words, v as 16 pairs in pairs_p4 order.
__device__ __forceinline__ float dot_chunk(const uint4 &w, const uint32_t (&v)[16]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float d0 = 0.f, d1 = 0.f;  // two chains of eight (half the dependent latency)
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float &d = (q & 1) ? d1 : d0;
      d = dot2_bf16(code_pair(ws[q], p), v[4 * q + p], d);
    }
  return d0 + d1;
}
constexpr uint32_t kOnes = 0x3f803f80u;  // the bf16 pair (1, 1)

__device__ __forceinline__ uint64_t tagged(uint32_t epoch, uint32_t v) { return ((uint64_t)epoch << 32) | v; }
__device__ __forceinline__ uint32_t tag_of(uint64_t r) { return (uint32_t)(r >> 32); }

struct DecShared {
  Sel64 S;
  uint32_t cand[kDecThreads / kWave][kMaxTopK];  // each wave's top-k keys
  int wcnt[kDecThreads / kWave];
  float wf[kDecThreads / kWave];
  double red[2][4];
  int ids[kMaxTopK];
  float gates[kMaxTopK];
  int fast;  // select_topk: the one-wave selection was certified
  float sgv;  // weight of the shared expert: sigmoid(x . w_sg), or 1
  float unit[kDnRows * kDnSlots];
  __attribute__((aligned(16))) uint32_t hb[kHStage / 32 * kHChunkWords];  // staged h, pairs_p4 order
  float hsum[kHStage / 32];  // sum of each staged chunk
};

// ------------------------------------------------------------------ router (binary64)

// Additions on any path of router_logit's sum: 8 per 2048 elements per lane, 6 levels
// across the wave, 3 across the four waves.
__device__ __forceinline__ int router_depth(int H) { return 8 * ((H + 2047) / 2048) + 9; }

// Binary64 logit of expert e (exact products, summed lane-sequentially, then over the
// wave, then over the four waves in order) and sum |x w|, in every thread.
// With set_ep, thread 0 also stores the call's tag (from the ticket tk, in flight until
// then) before the first barrier.
__device__ void router_logit(const DecodeArgs &a, DecShared &sh, int e, double &l, double &ab, bool set_ep,
                             uint64_t tk) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, H = a.H;
  double s = 0.0, sa = 0.0;
  for (int c = tid; c < H / 8; c += kDecThreads) {
    const uint4 xv = *(const uint4 *)(a.x + 8 * c);
    const float xf[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                         bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
    float wf[8];
    if (a.wr16) {
      const uint4 wv4 = *(const uint4 *)(a.wr16 + (size_t)e * H + 8 * c);
      wf[0] = bf16_lo(wv4.x); wf[1] = bf16_hi(wv4.x); wf[2] = bf16_lo(wv4.y); wf[3] = bf16_hi(wv4.y);
      wf[4] = bf16_lo(wv4.z); wf[5] = bf16_hi(wv4.z); wf[6] = bf16_lo(wv4.w); wf[7] = bf16_hi(wv4.w);
    } else {
      const float4 w0 = *(const float4 *)(a.wr32 + (size_t)e * H + 8 * c);
      const float4 w1 = *(const float4 *)(a.wr32 + (size_t)e * H + 8 * c + 4);
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
  s = wave_sum_f64(s);
  sa = wave_sum_f64(sa);
  if (lane == 0) {
    sh.red[0][wv] = s;
    sh.red[1][wv] = sa;
  }
  if (set_ep && tid < kWave) s_epoch = epoch_of(lane0_u64(tk));
  __syncthreads();
  l = ((sh.red[0][0] + sh.red[0][1]) + sh.red[0][2]) + sh.red[0][3];
  ab = ((sh.red[1][0] + sh.red[1][1]) + sh.red[1][2]) + sh.red[1][3];
  if (a.bias) l += (double)a.bias[e];
  __syncthreads();
}

// This workgroup's copy of the logit records.
__device__ __forceinline__ const uint64_t *lrec_copy(const DecodeArgs &a) {
  return a.lrec + (size_t)(blockIdx.x % kLrecRep) * a.E * 3;
}

// Wait for expert e's three logit records of this call.
__device__ void read_logit(const DecodeArgs &a, int e, double &v, double &r) {
  const uint64_t *rec = lrec_copy(a) + 3 * (size_t)e;
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

// Top-k of the E logits by one wave (four experts per lane): the keys of select_topk,
// k rounds of a wave maximum, the same certificate (every chosen logit minus its radius
// above every other logit plus its radius); ids ascending and softmax gates into sh.ids,
// sh.gates.  The lane's twelve records are loaded together and re-polled together.
// Returns false, having written nothing, when the certificate fails.
__device__ bool select_topk_wave(const DecodeArgs &a, DecShared &sh, bool write_debug) {
  constexpr int NV = kMaxExperts / kWave;
  const int lane = threadIdx.x & 63, E = a.E, k = a.k;
  double v[NV], r[NV];
  bool valid[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) valid[i] = lane + kWave * i < E;
  uint64_t rec[NV][3];
  const uint64_t *lr = lrec_copy(a);
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) rec[i][j] = valid[i] ? ld_agent(&lr[3 * (size_t)(lane + kWave * i) + j]) : 0u;
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
  // k rounds over the lanes' heads: each lane sorts its keys once (descending), a round
  // takes the wave maximum of the heads and the lane holding it (keys are distinct) moves
  // on to its next key.  The k-th winner is the threshold: an expert is chosen iff its
  // (nonzero) key is at least that.
  static_assert(NV == 4, "four keys per lane");
  uint32_t h0 = key[0], h1 = key[1], h2 = key[2], h3 = key[3];
  auto cx = [](uint32_t &x, uint32_t &y) {
    const uint32_t hi = max(x, y), lo = min(x, y);
    x = hi;
    y = lo;
  };
  cx(h0, h1); cx(h2, h3); cx(h0, h2); cx(h1, h3); cx(h1, h2);
  int top_e = 0;      // the first round's winner: the largest chosen logit
  uint32_t kth = 0;   // the last round's winner
  for (int rr = 0; rr < kMaxTopK; ++rr) {
    if (rr >= k) break;
    const uint32_t best = wave_max_u32(h0);
    const bool win = h0 == best;
    h0 = win ? h1 : h0;
    h1 = win ? h2 : h1;
    h2 = win ? h3 : h2;
    h3 = win ? 0u : h3;
    if (rr == 0) top_e = 255 - (int)(best & 0xffu);
    kth = best;
  }
  uint32_t chosen = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) chosen |= (key[i] != 0u && key[i] >= kth) ? (1u << i) : 0u;
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
  // softmax of the chosen logits (as fp32), ids ascending; the largest is top_e's
  const int ti = min(top_e >> 6, NV - 1);
  double tv = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) tv = ti == i ? v[i] : tv;
  const float gmax = (float)readlane_d(tv, top_e & 63);
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
      const int e = lane + kWave * i;
      const float g = ex[i] / den;
      sh.ids[pos] = e;
      sh.gates[pos] = g;
      if (write_debug && a.dbg_ids) a.dbg_ids[pos] = e;
      if (write_debug && a.dbg_gates) a.dbg_gates[pos] = g;
    }
    below += __popcll(bal);
  }
  return true;
}

// Top-k of the E logits of this call (value descending, index ascending) into sh.ids
// (ascending) and sh.gates: select_topk_wave, or when its certificate fails the
// four-wave path below.  One expert per thread (E <= 256): each wave takes its top k
// by k rounds of a wave maximum; a chosen candidate is one of the 4k whose rank among
// them is below k.  The choice is certified against the binary64 error radii; experts
// closer than their radii are re-ranked by resolve64.
__device__ void select_topk(const DecodeArgs &a, DecShared &sh, bool write_debug) {
  if (threadIdx.x < kWave) {
    const bool ok = select_topk_wave(a, sh, write_debug);
    if (threadIdx.x == 0) sh.fast = ok;
  }
  __syncthreads();
  if (sh.fast) return;  // uniform
  Sel64 &S = sh.S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, E = a.E, k = a.k;
  const bool mine = tid < E;
  double v = -INFINITY, r = 0.0;
  if (mine) {
    read_logit(a, tid, v, r);
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
    resolve64(S, k - nin1, a.x, a.wr16, a.wr32, a.bias, a.H, tid, kDecThreads);
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
    const float g = ex / den;
    sh.ids[below] = tid;
    sh.gates[below] = g;
    if (write_debug && a.dbg_ids) a.dbg_ids[below] = tid;
    if (write_debug && a.dbg_gates) a.dbg_gates[below] = g;
  }
  __syncthreads();
  if (tid < k) sh.ids[tid] = min(max(sh.ids[tid], 0), E - 1);  // keep reads in bounds even after a failed wait
  __syncthreads();
}

// ------------------------------------------------------------------ gate/up

// One round of a gate/up task for the calling wave: rows r0..r0+3 of slot j, the
// 32-element chunk c = lane + 64 p of the H-long rows.
struct GuLoad {
  uint4 wg[kGuRows], wu[kGuRows];
  uint2 sg, bg, su, bu;  // fp16 scale/bias of rows r0..r0+3: row r in half r%2 of word r/2
  uint4 x[4];
  bool ok;
};

__device__ __forceinline__ void gu_issue(const DecodeArgs &a, const QMat &Gm, const QMat &Um, int r0, int c,
                                         GuLoad &L) {
  const int H = a.H;
  L.ok = c < H / 32;
  const int cc = L.ok ? c : 0;
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    const size_t row = (size_t)(r0 + r);
    const size_t ci = code_index(row, 4 * cc, H);
    L.wg[r] = *(const uint4 *)(Gm.q + ci);
    L.wu[r] = *(const uint4 *)(Um.q + ci);
  }
  // r0 is a multiple of 4, so the four rows' values of one group are adjacent (8 bytes)
  const size_t qi = qp_index((size_t)r0, cc / 2, H / 64);
  L.sg = *(const uint2 *)(Gm.s + qi);
  L.bg = *(const uint2 *)(Gm.b + qi);
  L.su = *(const uint2 *)(Um.s + qi);
  L.bu = *(const uint2 *)(Um.b + qi);
#pragma unroll
  for (int q = 0; q < 4; ++q) L.x[q] = *(const uint4 *)(a.x + 32 * cc + 8 * q);
}

__device__ __forceinline__ void gu_accumulate(const GuLoad &L, bool bf, float (&ag)[kGuRows], float (&au)[kGuRows]) {
  if (!L.ok) return;
  uint32_t xp[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) pairs_p4(L.x[q].x, L.x[q].y, L.x[q].z, L.x[q].w, &xp[4 * q]);
  float xs = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) xs = dot2_bf16(kOnes, xp[i], xs);
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    auto half = [&](uint2 v) { return qp_f32(((r >> 1) ? v.y : v.x) >> (16 * (r & 1)), bf); };
    const float sg = half(L.sg), su = half(L.su);
    ag[r] += sg * dot_chunk(L.wg[r], xp) + (half(L.bg) - 128.0f * sg) * xs;
    au[r] += su * dot_chunk(L.wu[r], xp) + (half(L.bu) - 128.0f * su) * xs;
  }
}

__device__ __forceinline__ int gu_expert(const DecodeArgs &a, const DecShared &sh, int j) {
  return j < a.k ? sh.ids[j] : a.E;
}

__device__ __forceinline__ void gu_start(const DecodeArgs &a, const DecShared &sh, int g, GuLoad &L) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tpe = a.I / kGuTask;
  const int j = g / tpe, r0 = (g - j * tpe) * kGuTask + kGuRows * wv;
  const int e = gu_expert(a, sh, j);
  gu_issue(a, expert_mat(a.gate, a.s_gate, e, a.E, a.I, a.H), expert_mat(a.up, a.s_up, e, a.E, a.I, a.H), r0,
           lane, L);
}

// Gate/up task g: slot j = g / (I/16), rows i0 .. i0+15 (wave w: i0+4w .. i0+4w+3).
// `first` holds the already-issued first round.  Publishes this wave's 4 h records.
__device__ __forceinline__ void gu_task(const DecodeArgs &a, const DecShared &sh, int g, const GuLoad &first) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int I = a.I, H = a.H;
  const int tpe = I / kGuTask;
  const int j = g / tpe, r0 = (g - j * tpe) * kGuTask + kGuRows * wv;
  float ag[kGuRows] = {}, au[kGuRows] = {};
  gu_accumulate(first, a.qbf16, ag, au);
  const int np = (H / 32 + kWave - 1) / kWave;
  if (np > 1) {
    const int e = gu_expert(a, sh, j);
    const QMat Gm = expert_mat(a.gate, a.s_gate, e, a.E, I, H);
    const QMat Um = expert_mat(a.up, a.s_up, e, a.E, I, H);
    for (int p = 1; p < np; ++p) {
      GuLoad L;
      gu_issue(a, Gm, Um, r0, lane + kWave * p, L);
      gu_accumulate(L, a.qbf16, ag, au);
    }
  }
  float hv[kGuRows];  // uniform: the wave sums are read back to every lane
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    const float gs = wave_sum(ag[r]);
    const float us = wave_sum(au[r]);
    hv[r] = gs / (1.0f + __expf(-gs)) * us;
  }
  // rows r0 + 2p and r0 + 2p + 1 as one record (p = lane % 2): their h in bf16, the even
  // row in the low half, in kHrecRep copies (lane / 2), so fewer readers share a line
  const float h0 = (lane & 1) ? hv[2] : hv[0], h1 = (lane & 1) ? hv[3] : hv[1];
  const size_t pr = ((size_t)j * I + r0) / 2;
  if (lane < 2 * kHrecRep)
    st_agent(&a.hrec1[(size_t)(lane >> 1) * ((a.k + 1) * I / 2) + pr + (lane & 1)], tagged(s_epoch, pack_bf16x2(h0, h1)));
}

// ------------------------------------------------------------------ down

// u / nb for the small unit indices of a down round (u < 2^16 / nb): one 24-bit
// multiply and a shift with m = ceil(2^16 / nb), exact there, in place of a division by
// a runtime value (a long sequence of quarter-rate multiplies on the chain).
__device__ __forceinline__ int unit_div(int u, uint32_t m) { return (int)(__umul24((uint32_t)u, m) >> 16); }
__device__ __forceinline__ uint32_t unit_div_m(int nb) { return (65536u + (uint32_t)nb - 1u) / (uint32_t)nb; }

// Units of a down round: u = r * nb + jj (row r of the task, slot j0 + jj).  16-lane
// group q (lane/16 + 4*wave) takes u = q + 16 m; lane cl = lane % 16 takes the
// 32-element chunk c = cl + 16 p of the I-long rows.
struct DnLoad {
  uint4 w[kDnUnits];
  uint32_t s[kDnUnits], b[kDnUnits];
};

// routed = false: the selection may not have run in this workgroup; every slot reads the
// shared expert (loads whose results are discarded, from valid addresses).
__device__ __forceinline__ void dn_issue(const DecodeArgs &a, const DecShared &sh, int n0, int j0, int nb, int c,
                                         DnLoad &L, bool routed = true) {
  const int I = a.I, k = a.k, q = (threadIdx.x >> 4);
  const int cc = c < I / 32 ? c : 0;
  const uint32_t nbm = unit_div_m(nb);
#pragma unroll
  for (int m = 0; m < kDnUnits; ++m) {
    int u = q + 16 * m;
    u = u < kDnRows * nb ? u : 0;  // surplus units read unit 0 (result discarded)
    const int r = unit_div(u, nbm), slot = j0 + (u - r * nb);
    const int e = slot < k && routed ? sh.ids[slot] : a.E;
    const QMat D = expert_mat(a.down, a.s_down, e, a.E, a.H, I);
    const size_t n = (size_t)(n0 + r);
    L.w[m] = *(const uint4 *)(D.q + code_index(n, 4 * cc, I));
    const size_t qi = qp_index(n, cc / 2, I / 64);
    L.s[m] = D.s[qi];
    L.b[m] = D.b[qi];
  }
}

// h of slots j0 .. j0+nb-1 into LDS from their tagged records (two bf16 values each, in
// row order).  Thread t takes the 8-element groups g = t + 256 u, i.e. records 4g..4g+3:
// it loads all of its records at once and, while any is not yet tagged with this call's
// epoch, re-loads every such record together, so each round of the wait costs one
// memory round trip however many records were stale.  A group is stored regrouped for
// code_pair (pairs_p4) as words 4(g mod 4) .. 4(g mod 4)+3 of its 32-element chunk; then
// each chunk's sum.
__device__ __forceinline__ void stage_h(const DecodeArgs &a, DecShared &sh, int j0, int nb) {
  const int tid = threadIdx.x, I = a.I;
  const int ng = nb * I / 8;
  const uint64_t *rec = a.hrec1 + (size_t)(blockIdx.x % kHrecRep) * ((a.k + 1) * I / 2) + (size_t)j0 * I / 2;
  constexpr int kG = (kHStage / 8 + kDecThreads - 1) / kDecThreads;
  uint64_t rv[kG][4];
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int g = tid + u * kDecThreads;
#pragma unroll
    for (int r = 0; r < 4; ++r) rv[u][r] = g < ng ? ld_agent(&rec[4 * g + r]) : tagged(s_epoch, 0u);
  }
  for (int i = 0;; ++i) {
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kG; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) ok &= tag_of(rv[u][r]) == s_epoch;
    if (ok) break;
    if (i == kSpins) {
      st_agent(&a.ctrl->d_err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int g = tid + u * kDecThreads;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (g < ng && tag_of(rv[u][r]) != s_epoch) rv[u][r] = ld_agent(&rec[4 * g + r]);
    }
  }
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int g = tid + u * kDecThreads;
    if (g < ng) {
      uint32_t o[4];
      pairs_p4((uint32_t)rv[u][0], (uint32_t)rv[u][1], (uint32_t)rv[u][2], (uint32_t)rv[u][3], o);
      *(uint4 *)&sh.hb[(g >> 2) * kHChunkWords + 4 * (g & 3)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  __syncthreads();
  if (tid < nb * I / 32) {
    const uint4 *hp = (const uint4 *)&sh.hb[tid * kHChunkWords];
    float hs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = hp[i];
      hs = dot2_bf16(kOnes, v.x, hs);
      hs = dot2_bf16(kOnes, v.y, hs);
      hs = dot2_bf16(kOnes, v.z, hs);
      hs = dot2_bf16(kOnes, v.w, hs);
    }
    sh.hsum[tid] = hs;
  }
  __syncthreads();
}

__device__ __forceinline__ void dn_accumulate(const DecodeArgs &a, DecShared &sh, const DnLoad &L, int nb, int c,
                                              float (&acc)[kDnUnits]) {
  const int I = a.I, q = threadIdx.x >> 4;
  if (c >= I / 32) return;
  const uint32_t nbm = unit_div_m(nb);
#pragma unroll
  for (int m = 0; m < kDnUnits; ++m) {
    const int u = q + 16 * m;
    if (u >= kDnRows * nb) continue;
    const int ch = (u - unit_div(u, nbm) * nb) * (I / 32) + c;
    const uint4 *hp = (const uint4 *)&sh.hb[ch * kHChunkWords];
    uint32_t hv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = hp[i];
      hv[4 * i] = v.x;
      hv[4 * i + 1] = v.y;
      hv[4 * i + 2] = v.z;
      hv[4 * i + 3] = v.w;
    }
    const float sc = qp_f32(L.s[m], a.qbf16);
    acc[m] += sc * dot_chunk(L.w[m], hv) + (qp_f32(L.b[m], a.qbf16) - 128.0f * sc) * sh.hsum[ch];
  }
}

// Down task d: output rows n0 = 8d .. 8d+7 over every slot, rounds of nb slots and
// chunk passes; `pre` (if given) is round 0's first pass, already issued.
__device__ __forceinline__ void dn_task(const DecodeArgs &a, DecShared &sh, int d, const DnLoad &pre, bool has_pre) {
  const int tid = threadIdx.x, q = tid >> 4, cl = tid & 15;
  const int I = a.I, k = a.k, n0 = d * kDnRows;
  const int nbmax = min(min(k + 1, kDnSlots), kHStage / I);
  const int npass = (I / 32 + 15) / 16;
  float out_acc = 0.f;  // thread t < 8: row n0 + t
  for (int j0 = 0; j0 <= k; j0 += nbmax) {
    const int nb = min(nbmax, k + 1 - j0);
    const uint32_t nbm = unit_div_m(nb);
    stage_h(a, sh, j0, nb);
    float acc[kDnUnits] = {};
    for (int p = 0; p < npass; ++p) {
      const int c = cl + 16 * p;
      if (has_pre && j0 == 0 && p == 0) {
        dn_accumulate(a, sh, pre, nb, c, acc);
      } else {
        DnLoad L;
        dn_issue(a, sh, n0, j0, nb, c, L);
        dn_accumulate(a, sh, L, nb, c, acc);
      }
    }
#pragma unroll
    for (int m = 0; m < kDnUnits; ++m) {
      const float v = row16_sum(acc[m]);
      const int u = q + 16 * m;
      if (cl == 0 && u < kDnRows * nb) {
        const int slot = j0 + (u - unit_div(u, nbm) * nb);
        sh.unit[u] = (slot < k ? sh.gates[slot] : sh.sgv) * v;
      }
    }
    __syncthreads();
    if (tid < kDnRows)
      for (int jj = 0; jj < nb; ++jj) out_acc += sh.unit[tid * nb + jj];
    __syncthreads();
  }
  if (tid < kDnRows) a.out[n0 + tid] = f32_to_bf16(out_acc);
}

// ------------------------------------------------------------------ the layer

__global__ __launch_bounds__(kDecThreads) void k_decode1(DecodeArgs a) {
  __shared__ DecShared sh;
  const int b = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  // the call's ticket goes out now; thread 0 stores its tag to s_epoch in the first router
  // pass (or after the router loop) before any record is written or read
  // Thread 0's ticket is read back through lane 0 by all of wave 0 where it is used, so
  // the compiler neither moves that use up to the atomic nor copies the value where the
  // branch ends: either would wait for the atomic's round trip here.
  uint64_t tk;
  if (tid == 0) tk = epoch_ticket(a.epctr, kCtrStride / 2, b, G);
  const int E = a.E, k = a.k;
  const int n_gu = (k + 1) * (a.I / kGuTask), n_dn = a.H / kDnRows;
  const int first_shared = k * (a.I / kGuTask);  // gate/up tasks from here on are the shared expert's

  // The shared expert needs no routing: issue its gate/up loads before the router work.
  GuLoad gl;
  const bool gu_early = b < n_gu && b >= first_shared;
  if (gu_early) gu_start(a, sh, b, gl);

  // 1. router logits, published as records, kLrecRep copies of each (every workgroup
  // reads all of them, so the readers of one memory line are fewer)
  for (int e = b; e < E; e += G) {
    double l, ab;
    router_logit(a, sh, e, l, ab, e == b, tk);
    if (tid < 3 * kLrecRep) {
      const int w = tid % 3, cp = tid / 3;
      const uint64_t lb = (uint64_t)__double_as_longlong(l);
      const uint32_t v = w == 0 ? (uint32_t)lb
                       : w == 1 ? (uint32_t)(lb >> 32)
                                : __float_as_uint(__double2float_ru(radius64(l, ab, a.H, router_depth(a.H))));
      st_agent(&a.lrec[((size_t)cp * E + e) * 3 + w], tagged(s_epoch, v));
    }
  }
  if (b >= E) {
    if (tid < kWave) s_epoch = epoch_of(lane0_u64(tk));
    __syncthreads();
  }

  if (gu_early) gu_task(a, sh, b, gl);

  // 2. the selection, in every workgroup that uses it
  int g0 = gu_early ? b + G : b;
  const bool routed_gu = g0 < first_shared;
  if (routed_gu || b < n_dn || b == 0) select_topk(a, sh, b == 0);

  // 3. routed gate/up tasks; the first down task's loads go out with the first of them.
  // Both load groups are issued in straight-line code (the down loads unconditionally, from
  // a valid row), so the gate/up arithmetic waits for its own loads only: behind a branch,
  // the wait before the first use would cover every load issued on either path.
  DnLoad dl;
  bool dn_pre = false;
  const int nbmax = min(min(k + 1, kDnSlots), kHStage / a.I);
  if (g0 < n_gu) {
    gu_start(a, sh, g0, gl);
    dn_pre = b < n_dn;
    dn_issue(a, sh, min(b, n_dn - 1) * kDnRows, 0, min(nbmax, k + 1), tid & 15, dl, dn_pre);
    gu_task(a, sh, g0, gl);
    for (int g = g0 + G; g < n_gu; g += G) {
      gu_start(a, sh, g, gl);
      gu_task(a, sh, g, gl);
    }
  }

  // the shared expert's weight, in every workgroup with a down task: computed here, while
  // the h records are still on their way (at the start it delayed the router's loads)
  if (b < n_dn) {
    float z = 0.f;
    if (a.sgate) {
      for (int c = tid; c < a.H / 8; c += kDecThreads) {
        const uint4 xv = *(const uint4 *)(a.x + 8 * c), wv4 = *(const uint4 *)(a.sgate + 8 * c);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) z += bf16_lo(xw[i]) * bf16_lo(ww[i]) + bf16_hi(xw[i]) * bf16_hi(ww[i]);
      }
      z = wave_sum(z);
      if ((tid & 63) == 0) sh.wf[tid >> 6] = z;
    }
    __syncthreads();
    if (tid == 0) sh.sgv = a.sgate ? 1.0f / (1.0f + __expf(-((sh.wf[0] + sh.wf[1]) + (sh.wf[2] + sh.wf[3])))) : 1.0f;
    __syncthreads();
  }


  // 4. down tasks
  for (int d = b; d < n_dn; d += G) {
    dn_task(a, sh, d, dl, dn_pre);
    dn_pre = false;
  }
}

}  // namespace

int decode1_capacity(int n_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode1, kDecThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * n_cu;
}

int decode1_grid(const DecodeArgs &a, int capacity) {
  const int n_gu = (a.k + 1) * (a.I / kGuTask), n_dn = a.H / kDnRows;
  int want = a.E;
  want = want > n_gu ? want : n_gu;
  want = want > n_dn ? want : n_dn;
  return want < capacity ? want : capacity;
}

hipError_t launch_decode1(const DecodeArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_decode1, dim3(grid), dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
