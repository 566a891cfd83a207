// Gated DeltaNet prefill scan with the recurrent state resident in registers
// ("Optimizing on-device inference for Apple Silicon", section "Prefill > Keep
// recurrent state on chip": the state matrix is split by column, each column held in
// the registers of one SIMD group for the whole scan and written back once; partial
// results move between lanes, not through shared memory; state and gate in fp32,
// query and key in bf16).
//
// Update, per value head and token (the gated delta rule):
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
// Row j of S (one value channel, 128 fp32) is the "column" one 16-lane group owns:
// lane l holds elements 4l..4l+3 and 64+4l..64+4l+3.  A wave is four such groups
// (four channels), a workgroup four waves (16 channels of one value head).
//
// Per token the lanes form the partial dots s.k and s.q of the OLD row, reduce both
// over the 16 lanes with DPP butterflies (the same association in every lane, so all
// lanes hold bitwise equal sums), and then
//     c = beta (v_j - alpha s.k),   o_j = alpha s.q + c (k.q),   s <- alpha s + c k.
// The decay multiply is kept out of the per-element work: a lane stores s~ with
// s = A s~, where A is the product of the decays since the last renormalisation, so the
// update is one fma per element, s~ += (c / A') k with A' = alpha A.  The product is
// renormalised (folded into s~) at the first token of every 32-token block and whenever
// it would drop below 2^-64, so A' stays in [2^-64, 1] and 1/A' finite.
//
// Inputs are staged through LDS one 32-token block ahead: the workgroup converts the
// block's bf16 keys and queries to fp32 once (not once per channel), forms k.q per
// token, and computes the block's decay products; the next block's global loads are in
// flight while the current block is scanned.  Only the inputs pass through LDS; the
// state and the per-token reductions never do.
#include "kernels.hpp"
#include "common.hpp"

#pragma clang fp contract(off)

namespace moe {

namespace {

constexpr int kD = kGdnDim;             // 128
constexpr int kCols = 16;               // value channels per workgroup
constexpr int kTB = 32;                 // tokens per staged block
constexpr int kThreads = 256;
constexpr float kRenormBelow = 0x1p-64f;

struct GdnStage {
  float k[kTB][kD];
  float q[kTB][kD];
  float v[kCols][kTB];  // channel-major: one 16-byte read gives a channel 4 tokens
  float4 rec[kTB];      // A', beta, 1/A', k.q
  float pre[kTB];       // factor applied to s~ before the token (1: none)
  float pre0;           // pre[0]: the renormalisation at the block's first token
  int slow;             // the product was renormalised inside the block as well
};
// two staging buffers; the workgroup reserves more LDS than that so that no two
// workgroups share a compute unit (one wave per SIMD, the grid covers the chip once)
constexpr int kGdnLds = 96 * 1024;
static_assert(2 * sizeof(GdnStage) <= kGdnLds, "staging buffers exceed the reserved LDS");

__device__ __forceinline__ float dpp_sum16(float x) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: a butterfly
  // whose every step adds a value and its commuted partner, so all 16 lanes end equal
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ float dpp_sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  return x;
}

// The next block's inputs, held in registers while the current block is scanned.
// Thread (tt = tid / 8, p = tid % 8): keys and queries 16p..16p+15 of token tt, values
// 2p, 2p+1 of the workgroup's channels; threads of wave 0 with lane < 32 also hold the
// gates of token lane.
struct Prefetch {
  uint4 k0, k1, q0, q1;
  uint32_t v;
  float alpha, beta;
};

__device__ __forceinline__ void prefetch(const GdnArgs &a, int t0, int kh, int h, int c0, Prefetch &f) {
  const int tid = threadIdx.x, tt = tid >> 3, p = tid & 7;
  const int t = t0 + tt;
  if (t < a.T) {
    const uint4 *kp = (const uint4 *)(a.k + ((size_t)t * a.hk + kh) * kD + 16 * p);
    const uint4 *qp = (const uint4 *)(a.q + ((size_t)t * a.hk + kh) * kD + 16 * p);
    f.k0 = kp[0];
    f.k1 = kp[1];
    f.q0 = qp[0];
    f.q1 = qp[1];
    f.v = *(const uint32_t *)(a.v + ((size_t)t * a.hv + h) * kD + c0 + 2 * p);
  } else {
    f.k0 = f.k1 = f.q0 = f.q1 = make_uint4(0, 0, 0, 0);
    f.v = 0;
  }
  f.alpha = 1.0f;
  f.beta = 0.0f;
  if (tid < kTB && t0 + tid < a.T) {
    f.alpha = a.alpha[(size_t)(t0 + tid) * a.hv + h];
    f.beta = a.beta[(size_t)(t0 + tid) * a.hv + h];
  }
}

__device__ __forceinline__ void unpack8(uint4 w, float *o) {
  o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
  o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z); o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
}

// Write a prefetched block into LDS: fp32 keys, queries and values, k.q per token, and
// the decay records.  `carry` is A' of the last token before the block (1 at the start
// of the scan); returns A' of the block's last slot.
__device__ __forceinline__ float stage(const Prefetch &f, GdnStage &s, float carry) {
  const int tid = threadIdx.x, tt = tid >> 3, p = tid & 7;
  float kf[16], qf[16];
  unpack8(f.k0, kf);
  unpack8(f.k1, kf + 8);
  unpack8(f.q0, qf);
  unpack8(f.q1, qf + 8);
  float kq = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) kq = __builtin_fmaf(kf[e], qf[e], kq);
  kq = dpp_sum8(kq);
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    *(float4 *)&s.k[tt][16 * p + e] = make_float4(kf[e], kf[e + 1], kf[e + 2], kf[e + 3]);
    *(float4 *)&s.q[tt][16 * p + e] = make_float4(qf[e], qf[e + 1], qf[e + 2], qf[e + 3]);
  }
  s.v[2 * p][tt] = bf16_lo(f.v);
  s.v[2 * p + 1][tt] = bf16_hi(f.v);
  if (p == 0) s.rec[tt].w = kq;

  // decay products: wave 0, lane i < 32 holds token i's gates
  float last = carry;
  if (tid < 64) {
    const int i = tid;
    float x = (i == 0 || i >= kTB) ? 1.0f : f.alpha;
    // inclusive prefix product over lanes 0..31 (token 0 restarts the product: A' = 1)
#pragma unroll
    for (int d = 1; d < kTB; d <<= 1) {
      const float y = __shfl_up(x, d, 64);
      if (i >= d) x *= y;
    }
    const bool small = i < kTB && x < kRenormBelow;
    if (__ballot(small) == 0) {
      if (i < kTB) {
        const float pre = i == 0 ? carry * f.alpha : 1.0f;
        *(float3 *)&s.rec[i] = make_float3(x, f.beta, 1.0f / x);
        s.pre[i] = pre;
        if (i == 0) {
          s.pre0 = pre;
          s.slow = 0;
        }
      }
      last = __shfl(x, kTB - 1, 64);
    } else {
      // rare: a product would leave the range; walk the block in order instead (every
      // lane walks it, lane 0 writes the records)
      float A = 1.0f;
      for (int j = 0; j < kTB; ++j) {
        const float aj = __shfl(f.alpha, j, 64), bj = __shfl(f.beta, j, 64);
        float pre = 1.0f;
        if (j == 0) {
          pre = carry * aj;
          A = 1.0f;
        } else {
          A *= aj;
          if (A < kRenormBelow) {
            pre = A;
            A = 1.0f;
          }
        }
        if (i == 0) {
          *(float3 *)&s.rec[j] = make_float3(A, bj, 1.0f / A);
          s.pre[j] = pre;
        }
      }
      const float a0 = __shfl(f.alpha, 0, 64);
      if (i == 0) {
        s.pre0 = carry * a0;
        s.slow = 1;
      }
      last = A;
    }
  }
  return last;
}

// One token's inputs as one lane needs them.
struct TokIn {
  float4 r;               // A', beta, 1/A', k.q
  float4 k0, k1, q0, q1;  // elements 4l..4l+3 and 64+4l..64+4l+3
};

__device__ __forceinline__ TokIn load_tok(const GdnStage &s, int tt, int l) {
  TokIn x;
  x.r = s.rec[tt];
  x.k0 = *(const float4 *)&s.k[tt][4 * l];
  x.k1 = *(const float4 *)&s.k[tt][64 + 4 * l];
  x.q0 = *(const float4 *)&s.q[tt][4 * l];
  x.q1 = *(const float4 *)&s.q[tt][64 + 4 * l];
  return x;
}

// Scan one token: dots of the old row with k and q, their 16-lane sums, the write
// coefficient, the output and the row update; returns o_j.
__device__ __forceinline__ float scan_tok(const TokIn &x, float vj, float st[8]) {
  const float kv[8] = {x.k0.x, x.k0.y, x.k0.z, x.k0.w, x.k1.x, x.k1.y, x.k1.z, x.k1.w};
  const float qv[8] = {x.q0.x, x.q0.y, x.q0.z, x.q0.w, x.q1.x, x.q1.y, x.q1.z, x.q1.w};
  // two independent partial sums per dot halve the dependent chain
  float sk0 = st[0] * kv[0], sq0 = st[0] * qv[0], sk1 = st[4] * kv[4], sq1 = st[4] * qv[4];
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    sk0 = __builtin_fmaf(st[e], kv[e], sk0);
    sq0 = __builtin_fmaf(st[e], qv[e], sq0);
    sk1 = __builtin_fmaf(st[4 + e], kv[4 + e], sk1);
    sq1 = __builtin_fmaf(st[4 + e], qv[4 + e], sq1);
  }
  const float sk = dpp_sum16(sk0 + sk1);
  const float sq = dpp_sum16(sq0 + sq1);
  const float c = x.r.y * __builtin_fmaf(-x.r.x, sk, vj);  // beta (v - A' s~.k)
  const float o = __builtin_fmaf(x.r.x, sq, c * x.r.w);     // A' s~.q + c k.q
  const float d = c * x.r.z;                                // c / A'
#pragma unroll
  for (int e = 0; e < 8; ++e) st[e] = __builtin_fmaf(d, kv[e], st[e]);
  return o;
}

__global__ void __launch_bounds__(kThreads) k_gdn_scan(GdnArgs a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  GdnStage *stg = (GdnStage *)lds_raw;

  // workgroup -> (value head, channel block): the workgroups of one key head share an
  // XCD (workgroup b runs on XCD b % 8), so its keys and queries come from one L2
  const int nblk = kD / kCols;
  const int n_wg = a.hv * nblk;
  const int b = blockIdx.x;
  const int slot = (n_wg % kXcds == 0) ? (b % kXcds) * (n_wg / kXcds) + b / kXcds : b;
  const int h = slot / nblk, c0 = (slot % nblk) * kCols;
  const int kh = h / (a.hv / a.hk);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, l = lane & 15;
  const int col = wave * 4 + grp;  // channel within the workgroup
  const int j = c0 + col;

  // the row, scaled: s = A s~ (A = 1 here)
  float st[8];
  {
    const float *sp = a.state + ((size_t)h * kD + j) * kD;
    const float4 x0 = *(const float4 *)(sp + 4 * l);
    const float4 x1 = *(const float4 *)(sp + 64 + 4 * l);
    st[0] = x0.x; st[1] = x0.y; st[2] = x0.z; st[3] = x0.w;
    st[4] = x1.x; st[5] = x1.y; st[6] = x1.z; st[7] = x1.w;
  }

  Prefetch f;
  prefetch(a, 0, kh, h, c0, f);
  float carry = stage(f, stg[0], 1.0f);
  __syncthreads();

  float A = 1.0f;  // A' of the last scanned token
  const int nblocks = (a.T + kTB - 1) / kTB;
  for (int blk = 0; blk < nblocks; ++blk) {
    const int t0 = blk * kTB;
    if (blk + 1 < nblocks) prefetch(a, t0 + kTB, kh, h, c0, f);
    const GdnStage &s = stg[blk & 1];
    const int nt = min(kTB, a.T - t0);
    float keep = 0.0f;
    if (nt == kTB && !s.slow) {
      // a whole block without inner renormalisation: fully unrolled, every LDS offset and
      // every per-token decision fixed at compile time; a token's inputs are read two
      // tokens ahead.  With one wave per SIMD every instruction takes an issue slot of
      // its own (about 5.4 cycles per VALU instruction for a lone wave, measured), so the
      // loop keeps address arithmetic, branches and LDS reads out of the per-token path.
      const float pre = s.pre0;
#pragma unroll
      for (int e = 0; e < 8; ++e) st[e] *= pre;
      TokIn c0 = load_tok(s, 0, l), c1 = load_tok(s, 1, l);
      float4 v4 = *(const float4 *)&s.v[col][0];
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt) {
        TokIn c2;
        if (tt + 2 < kTB) c2 = load_tok(s, tt + 2, l);
        float4 v4n;
        if ((tt & 3) == 3 && tt + 1 < kTB) v4n = *(const float4 *)&s.v[col][tt + 1];
        const float vj = (tt & 3) == 0 ? v4.x : (tt & 3) == 1 ? v4.y : (tt & 3) == 2 ? v4.z : v4.w;
        const float o = scan_tok(c0, vj, st);
        if (l == (tt & 15)) keep = o;
        if ((tt & 15) == 15) a.out[((size_t)(t0 + (tt & ~15) + l) * a.hv + h) * kD + j] = f32_to_bf16(keep);
        c0 = c1;
        if (tt + 2 < kTB) c1 = c2;
        if ((tt & 3) == 3 && tt + 1 < kTB) v4 = v4n;
      }
      A = s.rec[kTB - 1].x;
    } else {
      // general block: a ragged last block, or renormalisations inside the block
      TokIn ta = load_tok(s, 0, l);
      for (int tt = 0; tt < nt; ++tt) {
        const TokIn tb = load_tok(s, min(tt + 1, kTB - 1), l);
        const int pre_bits = __builtin_amdgcn_readfirstlane(__float_as_int(s.pre[tt]));  // uniform
        if (pre_bits != 0x3f800000) {
          const float pre = __int_as_float(pre_bits);
#pragma unroll
          for (int e = 0; e < 8; ++e) st[e] *= pre;
        }
        const float o = scan_tok(ta, s.v[col][tt], st);
        A = ta.r.x;
        if (l == (tt & 15)) keep = o;
        if ((tt & 15) == 15 || tt == nt - 1) {
          const int tb0 = t0 + (tt & ~15);
          if (l <= (tt & 15)) a.out[((size_t)(tb0 + l) * a.hv + h) * kD + j] = f32_to_bf16(keep);
        }
        ta = tb;
      }
    }
    if (blk + 1 < nblocks) carry = stage(f, stg[(blk + 1) & 1], carry);
    __syncthreads();
  }

  {
    float *sp = a.state + ((size_t)h * kD + j) * kD;
    *(float4 *)(sp + 4 * l) = make_float4(A * st[0], A * st[1], A * st[2], A * st[3]);
    *(float4 *)(sp + 64 + 4 * l) = make_float4(A * st[4], A * st[5], A * st[6], A * st[7]);
  }
}

}  // namespace

hipError_t launch_gdn_scan(const GdnArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)k_gdn_scan, hipFuncAttributeMaxDynamicSharedMemorySize, kGdnLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_wg = a.hv * (kD / kCols);
  hipLaunchKernelGGL(k_gdn_scan, dim3(n_wg), dim3(kThreads), kGdnLds, s, a);
  return hipGetLastError();
}

}  // namespace moe
