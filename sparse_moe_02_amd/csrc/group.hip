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
// Block map: an expert with n rows is split into ceil(n/128) M-blocks of balanced height
// (section "Prefill > Match tile size to expert load": the tile height follows the
// expert's actual row count); each M-block records its height in 32-row MFMA tiles.
// Empty experts emit nothing, so their weights are never read.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void k_group(GroupArgs a) {
  __shared__ int s_cnt[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 2];
  __shared__ int s_cls[5];     // M-blocks per tile-height class (1..4 tiles of 32 rows)
  __shared__ int s_clsoff[5];
  __shared__ int s_clspos[5];
  const int tid = threadIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int nblk = (T + kRouteTokens - 1) / kRouteTokens;

  // 1. histogram and per-workgroup bases (thread per expert, sequential over workgroups)
  if (tid < E) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      a.base[(size_t)b * E + tid] = run;
      run += __popc(a.tokmask[(size_t)b * E + tid]);
    }
    s_cnt[tid] = run;
  }
  if (tid == E) s_cnt[E] = T;
  if (tid < 5) {
    s_cls[tid] = 0;
    s_clspos[tid] = 0;
  }
  __syncthreads();

  // 2. exclusive prefix scan over the E+1 bins (one wave; lane takes a contiguous run)
  if (tid < kWave) {
    const int per = (E + 1 + kWave - 1) / kWave;
    const int lo = tid * per, hi = min(lo + per, E + 1);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += s_cnt[e];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    int run = incl - sum;
    for (int e = lo; e < hi; ++e) {
      s_off[e] = run;
      run += s_cnt[e];
    }
    if (tid == kWave - 1) s_off[E + 1] = incl;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kThreads) {
    a.counts[e] = s_cnt[e];
    if (a.dbg_counts) a.dbg_counts[e] = s_cnt[e];
  }
  for (int e = tid; e <= E + 1; e += kThreads) {
    a.offsets[e] = s_off[e];
    if (a.dbg_offsets) a.dbg_offsets[e] = s_off[e];
  }

  // 3. scatter: grouped row of every (token, chosen expert) and of the shared slot
  for (int t = tid; t < T; t += kThreads) {
    const int b = t / kRouteTokens;
    const uint32_t below = (1u << (t % kRouteTokens)) - 1u;
    for (int j = 0; j < k; ++j) {
      const int e = a.ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;  // cannot happen for router output
      const size_t be = (size_t)b * E + e;
      const int pos = s_off[e] + a.base[be] + __popc(a.tokmask[be] & below);
      if (pos < s_off[e] || pos >= s_off[e + 1]) continue;
      a.row_token[pos] = t;
      a.row_gate[pos] = a.gates[(size_t)t * k + j];
      if (a.dbg_row_token) a.dbg_row_token[pos] = t;
    }
    const int pos = s_off[E] + t;
    a.row_token[pos] = t;
    a.row_gate[pos] = 1.0f;
    if (a.dbg_row_token) a.dbg_row_token[pos] = t;
  }

  // 4. block map: balanced M-blocks per expert, ordered tallest class first
  int nmb = 0, q = 0, rem = 0;
  if (tid <= E) {
    const int n = s_cnt[tid];
    nmb = (n + kBM - 1) / kBM;
    if (nmb) {
      q = n / nmb;
      rem = n % nmb;
      // rem blocks of q+1 rows, nmb-rem blocks of q rows
      if (rem) atomicAdd(&s_cls[(q + 1 + 31) / 32], rem);
      if (nmb - rem) atomicAdd(&s_cls[(q + 31) / 32], nmb - rem);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 4; c >= 1; --c) {
      s_clsoff[c] = run;
      run += s_cls[c];
    }
    a.ctrl->n_mblocks = run;
    a.ctrl->q_gateup = 0;
    a.ctrl->q_down = 0;
    if (a.dbg_n_refined) *a.dbg_n_refined = a.ctrl->n_refined;
    a.ctrl->n_refined = 0;
  }
  __syncthreads();
  if (tid <= E && nmb) {
    int row = s_off[tid];
    for (int i = 0; i < nmb; ++i) {
      const int rows = q + (i < rem ? 1 : 0);
      const int cls = (rows + 31) / 32;
      const int slot = s_clsoff[cls] + atomicAdd(&s_clspos[cls], 1);
      a.mblocks[slot] = make_int4(tid, row, rows, cls);
      row += rows;
    }
  }
}

}  // namespace

hipError_t launch_group(const GroupArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_group, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
