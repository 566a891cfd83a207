// Decode form (one token): row-parallel dequant-GEMV over the k routed experts and the
// shared expert, no MFMA.
//
// "Optimizing on-device inference for Apple Silicon", section "Decode > Optimize the
// one-row weight path": a group of lanes cooperates on one output while reading
// different parts of the weight row in parallel.  Section "Decode > Reduce intermediate
// and state traffic": the two input projections and the gated activation form one
// kernel; the output projection, the routing weights and the shared expert's result form
// another.  Batch-1 decode moves every active weight byte once, so both kernels are
// bound by HBM reads: each lane issues 16-byte loads of packed codes and the dot product
// is taken against the codes directly,
//     sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k   (per group of 64),
// in fp32, then reduced across the lanes of the row.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGuRows = 4;   // gate/up rows per wave
constexpr int kDnRows = 16;  // output rows per down workgroup

__device__ __forceinline__ QMat expert_mat(const QMat &routed, const QMat &shared, int e, int E, int N, int K) {
  if (e == E) return shared;
  QMat m;
  m.q = routed.q + (size_t)e * N * (K / 8);
  m.s = routed.s + (size_t)e * N * (K / 64);
  m.b = routed.b + (size_t)e * N * (K / 64);
  return m;
}

// sum_i v[i] * code_i over the 32 codes of four packed words
__device__ __forceinline__ float dot_codes32(const uint4 &w, const float (&v)[32]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t lo = ws[q] & 0x0f0f0f0fu, hi = (ws[q] >> 4) & 0x0f0f0f0fu;
    asm("" : "+v"(lo), "+v"(hi));  // one v_cvt_f32_ubyteN per code
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = __builtin_fmaf(v[8 * q + 2 * j], (float)((lo >> (8 * j)) & 0xffu), s);
      s = __builtin_fmaf(v[8 * q + 2 * j + 1], (float)((hi >> (8 * j)) & 0xffu), s);
    }
  }
  return s;
}

// Gate/up for expert slot j (j < k: routed ids[j]; j == k: shared), rows i0..i0+3.
// Lane takes 32-element chunks c = lane + 64 p of the H-long rows.
__global__ __launch_bounds__(64) void k_decode_gateup(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int H = a.H, I = a.I, E = a.E, k = a.k;
  const int per = I / kGuRows;
  const int j = blockIdx.x / per;
  const int i0 = (blockIdx.x - j * per) * kGuRows;
  const int e = j < k ? a.ids[j] : E;
  const QMat G = expert_mat(a.gate, a.s_gate, e, E, I, H);
  const QMat U = expert_mat(a.up, a.s_up, e, E, I, H);
  float accg[kGuRows] = {}, accu[kGuRows] = {};
  for (int c = lane; c < H / 32; c += kWave) {
    uint4 wg[kGuRows], wu[kGuRows];
    float sg[kGuRows], bg[kGuRows], su[kGuRows], bu[kGuRows];
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) {
      const size_t row = (size_t)(i0 + r);
      wg[r] = *(const uint4 *)(G.q + row * (H / 8) + 4 * c);
      wu[r] = *(const uint4 *)(U.q + row * (H / 8) + 4 * c);
      sg[r] = fp16_to_f32(G.s[row * (H / 64) + c / 2]);
      bg[r] = fp16_to_f32(G.b[row * (H / 64) + c / 2]);
      su[r] = fp16_to_f32(U.s[row * (H / 64) + c / 2]);
      bu[r] = fp16_to_f32(U.b[row * (H / 64) + c / 2]);
    }
    float xf[32];
    float xs = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = *(const uint4 *)(a.x + 32 * c + 8 * q);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xf[8 * q + 2 * i] = bf16_lo(xw[i]);
        xf[8 * q + 2 * i + 1] = bf16_hi(xw[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) xs += xf[i];
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) {
      accg[r] += sg[r] * dot_codes32(wg[r], xf) + bg[r] * xs;
      accu[r] += su[r] * dot_codes32(wu[r], xf) + bu[r] * xs;
    }
  }
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    const float g = wave_sum(accg[r]);
    const float u = wave_sum(accu[r]);
    if (lane == 0) a.hbuf[(size_t)j * I + i0 + r] = g / (1.0f + __expf(-g)) * u;
  }
}

// Down + combine: out[n] = sum_{j<k} gates[j] * Wd_{ids[j]}[n,:] . h_j + Wd_s[n,:] . h_k.
// One workgroup of min(k+1, 16) waves per kDnRows output rows; wave j owns expert slot j
// (and j + 16), keeps
// its 32-element chunk of h_j in registers and issues all its weight loads at once.
// LPR lanes share a row (32 codes each); per-slot partial sums meet in LDS.
template <int LPR>
__global__ __launch_bounds__(1024) void k_decode_down(DecodeArgs a) {
  constexpr int RPP = kWave / LPR;           // rows per pass
  constexpr int P = kDnRows / RPP;           // passes (kDnRows is a multiple of RPP)
  __shared__ float s_part[kMaxTopK + 1][kDnRows];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int H = a.H, I = a.I, E = a.E, k = a.k;
  const int sub = lane / LPR, cl = lane % LPR;
  const int n0 = blockIdx.x * kDnRows;
  for (int j = wv; j <= k; j += nw) {
    const int e = j < k ? a.ids[j] : E;
    const float gj = j < k ? a.gates[j] : 1.0f;
    const QMat D = expert_mat(a.down, a.s_down, e, E, H, I);
    float acc[P] = {};
    for (int c = cl; c < I / 32; c += LPR) {
      uint4 w[P];
      float sc[P], bi[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const size_t n = (size_t)(n0 + p * RPP + sub);
        w[p] = *(const uint4 *)(D.q + n * (I / 8) + 4 * c);
        sc[p] = fp16_to_f32(D.s[n * (I / 64) + c / 2]);
        bi[p] = fp16_to_f32(D.b[n * (I / 64) + c / 2]);
      }
      float hv[32];
      const float4 *hp = (const float4 *)(a.hbuf + (size_t)j * I + 32 * c);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = hp[q];
        hv[4 * q] = v.x;
        hv[4 * q + 1] = v.y;
        hv[4 * q + 2] = v.z;
        hv[4 * q + 3] = v.w;
      }
      float hs = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) hs += hv[i];
#pragma unroll
      for (int p = 0; p < P; ++p) acc[p] += sc[p] * dot_codes32(w[p], hv) + bi[p] * hs;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float v = acc[p];
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o);
      if (cl == 0) s_part[j][p * RPP + sub] = gj * v;
    }
  }
  __syncthreads();
  if (threadIdx.x < kDnRows) {
    float v = 0.f;
    for (int jj = 0; jj <= k; ++jj) v += s_part[jj][threadIdx.x];
    a.out[n0 + threadIdx.x] = f32_to_bf16(v);
  }
}

}  // namespace

hipError_t launch_decode_gateup(const DecodeArgs &a, hipStream_t s) {
  const int nb = (a.k + 1) * (a.I / kGuRows);
  hipLaunchKernelGGL(k_decode_gateup, dim3(nb), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs &a, hipStream_t s) {
  const int cpr = a.I / 32;
  const int lpr = cpr < kWave ? cpr : kWave;
  const int nw = a.k + 1 < 16 ? a.k + 1 : 16;  // waves; each loops over its expert slots
  const dim3 grid(a.H / kDnRows), block(64 * nw);
  switch (lpr) {
    case 4: hipLaunchKernelGGL(k_decode_down<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_decode_down<8>, grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL(k_decode_down<16>, grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL(k_decode_down<32>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_decode_down<64>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
