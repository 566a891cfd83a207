// Grouping of routed rows by expert, entirely on the device.
//
// "Optimizing on-device inference for Apple Silicon", section "Prefill > Keep expert
// routing on the GPU": a histogram counts the assignments of each expert, a prefix scan
// turns the counts into start offsets, a scatter places every routed row in its
// expert's group, and a block map lists the matrix blocks the grouped GEMMs process.
//
// The router leaves, per 32-token workgroup b and expert e, a bit mask of the tokens of
// b that chose e.  Counts are popcounts; a token's rank inside its expert group is the
// count of earlier workgroups plus the popcount of the earlier bits of its own mask, so
// rows of an expert are in ascending token order without atomics.  Bin E is the shared
// expert, which every token visits.
//
// One workgroup per 64 tokens; each rereads every mask (popcounts are cheap), so no
// workgroup waits for another (at 4096 tokens, 64 workgroups measured 12.3 us for the
// stage against 14.7 us with 16 workgroups of 256 tokens).  Every global read the
// workgroup needs (all masks, and the ids and gates of its own tokens) is issued before
// the first is used, so the kernel pays one memory latency.
//
// Block map: an expert with n rows is split into ceil(n/160) M-blocks of balanced height
// (section "Prefill > Match tile size to expert load": the tile height follows the
// expert's actual row count); each M-block records its height in 32-row MFMA tiles.
// Empty experts emit nothing, so their weights are never read.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kSubs = 2;                                 // router workgroups per group workgroup
constexpr int kTokensPerBlock = kSubs * kRouteTokens;   // 64
constexpr int kQuads = kMaxExperts / 4;                 // four experts per 16-byte mask load
constexpr int kParts = kThreads / kQuads;               // 16 threads per four-expert column

// Workgroup g handles tokens [64 g, 64 g + 64) = router workgroups 2g, 2g+1.  Every
// workgroup reads all bit masks to get the expert totals (hence the offsets) and the
// count of earlier tokens per expert; workgroup 0 also writes the offsets and the block
// map and resets the work queues.
constexpr int kScat = (kTokensPerBlock * (kMaxTopK + 1) + kThreads - 1) / kThreads;  // scatter items per thread
constexpr int kBatch = 8;                               // 16-byte mask loads in flight per thread

__global__ __launch_bounds__(kThreads) void k_group(GroupArgs a) {
  __shared__ int s_tot[kParts][kMaxExperts];
  __shared__ int s_pre[kParts][kMaxExperts];
  static_assert(sizeof(int) * kParts * kMaxExperts * 2 <= 32768, "count tables");
  __shared__ int s_off[kMaxExperts + 2];
  __shared__ int s_cnt[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) uint32_t s_msk[kSubs][kMaxExperts];
  __shared__ int s_base[kSubs][kMaxExperts];
  __shared__ int s_cls[6], s_clsoff[6];
  __shared__ int s_pc[kBM / 32 + 1][kMaxExperts + 1];  // per class, per expert: M-blocks (then their scan)
  __shared__ int s_mbs[kMaxExperts + 2];                // M-blocks of the experts before e (all classes)
  const int tid = threadIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int nblk = (T + kRouteTokens - 1) / kRouteTokens;
  const int sb0 = blockIdx.x * kSubs;
  const int t0 = blockIdx.x * kTokensPerBlock;
  const uint32_t *__restrict__ mask = a.tokmask;

  // 0. the expert ids and gates this thread scatters in step 3 (loads issued now)
  int sc_e[kScat];
  float sc_g[kScat];
#pragma unroll
  for (int u = 0; u < kScat; ++u) {
    const int i = tid + u * kThreads;
    const int lt = i / (k + 1), j = i - lt * (k + 1);
    const int t = t0 + lt;
    const bool ld = lt < kTokensPerBlock && t < T && j < k;
    sc_e[u] = ld ? a.ids[(size_t)t * k + j] : -1;
    sc_g[u] = ld ? a.gates[(size_t)t * k + j] : 1.0f;
  }

  // 1. per expert: total count, and count over router workgroups before sb0; the masks
  // of this workgroup's own router workgroups are kept for the ranks.  Thread (q, part)
  // reads experts 4q..4q+3 of router workgroups part, part+16, ... (rows are 256 words,
  // zero past E).
  {
    const int q = tid % kQuads, part = tid / kQuads;
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    for (int b0 = part; b0 < nblk; b0 += kParts * kBatch) {
      uint4 mv[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int b = b0 + kParts * i;
        mv[i] = b < nblk ? *(const uint4 *)(mask + (size_t)b * kMaxExperts + 4 * q) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int b = b0 + kParts * i;
        const uint32_t w[4] = {mv[i].x, mv[i].y, mv[i].z, mv[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = __popc(w[c]);
          tot[c] += n;
          pre[c] += b < sb0 ? n : 0;
        }
        if (b >= sb0 && b < sb0 + kSubs) *(uint4 *)&s_msk[b - sb0][4 * q] = mv[i];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s_tot[part][4 * q + c] = tot[c];
      s_pre[part][4 * q + c] = pre[c];
    }
  }
  for (int i = tid; i < kSubs * kMaxExperts; i += kThreads) {
    const int j = i / kMaxExperts;
    if (sb0 + j >= nblk) s_msk[j][i % kMaxExperts] = 0u;
  }
  if (tid < 6) {
    s_cls[tid] = 0;
  }
  __syncthreads();
  if (tid < E) {
    int tot = 0;
    for (int p = 0; p < kParts; ++p) tot += s_tot[p][tid];
    s_cnt[tid] = tot;
  }
  if (tid == E) s_cnt[E] = T;
  __syncthreads();

  // 2. exclusive prefix scan over the E+1 bins (one wave; lane takes a contiguous run)
  if (tid < kWave) {
    const int per = (E + 1 + kWave - 1) / kWave;
    const int lo = tid * per, hi = min(lo + per, E + 1);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += s_cnt[e];
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
    for (int e = lo; e < hi; ++e) {
      s_off[e] = run;
      run += s_cnt[e];
    }
    if (tid == kWave - 1) s_off[E + 1] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int run = s_off[tid];
    for (int p = 0; p < kParts; ++p) run += s_pre[p][tid];
    for (int j = 0; j < kSubs; ++j) {
      s_base[j][tid] = run;
      run += __popc(s_msk[j][tid]);
    }
  }
  __syncthreads();

  // 3. scatter: grouped row of every (token, chosen expert) and of the shared slot
#pragma unroll
  for (int u = 0; u < kScat; ++u) {
    const int i = tid + u * kThreads;
    const int lt = i / (k + 1), j = i - lt * (k + 1);
    const int t = t0 + lt;
    if (lt >= kTokensPerBlock || t >= T) continue;
    int pos;
    float g;
    if (j < k) {
      const int e = sc_e[u];
      if ((unsigned)e >= (unsigned)E) continue;  // cannot happen for router output
      const int sj = lt / kRouteTokens;
      const uint32_t below = (1u << (lt % kRouteTokens)) - 1u;
      pos = s_base[sj][e] + __popc(s_msk[sj][e] & below);
      if (pos < s_off[e] || pos >= s_off[e + 1]) continue;
      g = sc_g[u];
    } else {
      pos = s_off[E] + t;
      g = a.sgate ? a.sgate[t] : 1.0f;
    }
    a.row_token[pos] = t;
    a.row_gate[pos] = g;
    a.slot_row[(size_t)t * (k + 1) + j] = pos;
    if (a.dbg_row_token) a.dbg_row_token[pos] = t;
  }
  if (blockIdx.x != 0) return;

  for (int e = tid; e <= E; e += kThreads) {
    a.counts[e] = s_cnt[e];
    if (a.dbg_counts) a.dbg_counts[e] = s_cnt[e];
  }
  for (int e = tid; e <= E + 1; e += kThreads) {
    a.offsets[e] = s_off[e];
    if (a.dbg_offsets) a.dbg_offsets[e] = s_off[e];
  }

  // 4. block map: balanced M-blocks per expert, ordered tallest class first.  With a
  // forced height F: floor(n/F) blocks of F rows and one block of the remainder.  Inside
  // a height class the blocks follow in expert order (a prefix scan over the experts'
  // block counts of that class, not an atomic), so the map, and with it the items the
  // gate/up GEMM splits along K, is the same on every run.
  constexpr int kCls = kBM / 32;
  int nmb = 0, q = 0, rem = 0;
  const int F = a.force_rows;
  for (int i = tid; i < (kCls + 1) * (kMaxExperts + 1); i += kThreads) (&s_pc[0][0])[i] = 0;
  __syncthreads();
  if (tid <= E) {
    const int n = s_cnt[tid];
    if (F) {
      nmb = (n + F - 1) / F;
      if (nmb) {
        q = F;
        rem = n - (nmb - 1) * F;  // rows of the last block (1..F)
        if (nmb > 1) s_pc[F / 32][tid] += nmb - 1;
        s_pc[(rem + 31) / 32][tid] += 1;
      }
    } else {
      nmb = (n + kBM - 1) / kBM;
      if (nmb) {
        q = n / nmb;
        rem = n % nmb;
        // rem blocks of q+1 rows, nmb-rem blocks of q rows
        if (rem) s_pc[(q + 1 + 31) / 32][tid] += rem;
        if (nmb - rem) s_pc[(q + 31) / 32][tid] += nmb - rem;
      }
    }
  }
  __syncthreads();
  // exclusive scan of each class's per-expert counts (wave c-1 takes class c); the total
  // goes to s_cls[c]
  if (tid < kCls * kWave) {
    const int c = tid / kWave + 1, lane = tid % kWave;
    const int per = (E + 1 + kWave - 1) / kWave;
    const int lo = lane * per, hi = min(lo + per, E + 1);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += s_pc[c][e];
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
    for (int e = lo; e < hi; ++e) {
      const int v = s_pc[c][e];
      s_pc[c][e] = run;
      run += v;
    }
    if (lane == kWave - 1) s_cls[c] = incl;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = kCls; c >= 1; --c) {
      s_clsoff[c] = run;
      run += s_cls[c];
    }
    a.ctrl->n_mblocks = run;
    for (int x = 0; x < kXcds; ++x) {
      a.ctrl->q_gateup[x] = 0;
      a.ctrl->q_down[x] = 0;
    }
    a.ctrl->q_tail = 0;
    if (a.dbg_n_refined) *a.dbg_n_refined = a.ctrl->n_refined;
    a.ctrl->n_refined = 0;
  }
  // every M-block placed by a thread of its own (the shared expert alone has T/160 of
  // them): flat block index f -> its expert e (the last with s_mbs[e] <= f) and index i
  // inside e; blocks of one class keep their order inside the expert
  if (tid <= E) {
    int before = 0;
#pragma unroll
    for (int c = 1; c <= kCls; ++c) before += s_pc[c][tid];
    s_mbs[tid] = before;
  }
  if (tid == 0) s_mbs[E + 1] = s_clsoff[1] + s_cls[1];  // every block (class 1 comes last)
  __syncthreads();
  const int n_all = s_mbs[E + 1];
  for (int f = tid; f < n_all; f += kThreads) {
    int lo = 0, hi = E;  // s_mbs[lo] <= f < s_mbs[hi + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_mbs[mid] <= f)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int e = lo, i = f - s_mbs[e], n = s_cnt[e];
    int rows, row, pos;
    if (F) {
      const int nb = (n + F - 1) / F, last = n - (nb - 1) * F;
      rows = i + 1 < nb ? F : last;
      row = s_off[e] + i * F;
      // the full blocks come first; the last one is first of its class unless it is full
      pos = (i + 1 < nb || (last + 31) / 32 == F / 32) ? i : 0;
    } else {
      const int nb = (n + kBM - 1) / kBM, qq = n / nb, rr = n % nb;
      rows = qq + (i < rr ? 1 : 0);
      row = s_off[e] + i * qq + min(i, rr);
      // rr blocks of qq+1 rows, then nb-rr of qq rows: one class, or two in that order
      pos = ((qq + 1 + 31) / 32 == (qq + 31) / 32 || i < rr) ? i : i - rr;
    }
    const int cls = (rows + 31) / 32;
    a.mblocks[s_clsoff[cls] + s_pc[cls][e] + pos] = make_int4(e, row, rows, cls);
  }
}

// The shared expert's weight per token, sigmoid(x_t . w) with w the learned gate vector:
// one wave per token, each lane 8-element chunks c = lane + 64 i, bf16 products summed in
// fp32 (v_dot2), then the wave sum.
__global__ __launch_bounds__(256) void k_shared_gate(const uint16_t *x, const uint16_t *w, float *out, int T, int H) {
  const int lane = threadIdx.x & 63, t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  float z = 0.f;
  for (int c = lane; c < H / 8; c += kWave) {
    const uint4 xv = *(const uint4 *)(x + (size_t)t * H + 8 * c), wv = *(const uint4 *)(w + 8 * c);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xw[i]), __builtin_bit_cast(bf16x2, ww[i]), z,
                                          false);
  }
  z = wave_sum(z);
  if (lane == 0) out[t] = 1.0f / (1.0f + __expf(-z));
}

}  // namespace

hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *w, float *out, int T, int H, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gate, dim3((T + 3) / 4), dim3(256), 0, s, x, w, out, T, H);
  return hipGetLastError();
}

hipError_t launch_group(const GroupArgs &a, hipStream_t s) {
  const int nb = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(k_group, dim3(nb), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
