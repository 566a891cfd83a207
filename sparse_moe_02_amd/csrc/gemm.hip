// Grouped GEMMs of the prefill form, bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation and int4 weights dequantised on chip.
//
// "Optimizing on-device inference for Apple Silicon", section "Prefill > Dequantize
// weights during matmul": the grouped GEMM reconstructs one small weight tile at a time
// in on-chip memory and multiplies it with the routed activation rows, accumulating in
// fp32; the expanded weight array never exists in memory.  Section "Decode > Reduce
// intermediate and state traffic" fuses the gated activation with the input
// projections and the routing score and shared expert with the output projection; the
// same fusions are applied here: SwiGLU in the gate/up epilogue, gate-weighted
// scatter-add in the down epilogue.
//
// MI355X mapping.  A work item is (M-block of one expert, N-block).  Four waves split
// the N-block; each wave covers all rows of the M-block (1..4 tiles of 32), so a weight
// element is dequantised once per work item.  For a 128-wide K super-step, lane l of a
// wave owns weight row n = l%32 and the 64 consecutive k of half h = l/32: exactly eight
// packed words and one (scale, bias) pair.  Word j feeds MFMA j of the super-step, whose
// B operand wants 8 consecutive k per lane; the activation operand uses the same k
// assignment (k = 64h + 8j + i), so any k order inside the super-step is consistent.
// Activation rows (gathered by token for gate/up, contiguous h rows for down) are staged
// in LDS, double buffered, with the 16-byte chunk index XOR-swizzled by row.
// Work items are handed out by an atomic queue (persistent grid), tallest M-blocks first.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRowBytes = 256;                      // 128 bf16 per staged row
constexpr int kBufBytes = kBM * kRowBytes;          // one LDS buffer (32 KiB)

__device__ __forceinline__ QMat expert_mat(const QMat &routed, const QMat &shared, int e, int E, int N,
                                           int K) {
  if (e == E) return shared;
  QMat m;
  m.q = routed.q + (size_t)e * N * (K / 8);
  m.s = routed.s + (size_t)e * N * (K / 64);
  m.b = routed.b + (size_t)e * N * (K / 64);
  return m;
}

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 15)) << 4); }

__device__ __forceinline__ uint32_t word_of(const uint4 &lo, const uint4 &hi, int j) {
  const uint4 &v = j < 4 ? lo : hi;
  const int i = j & 3;
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const uint32_t (&b)[4], const f32x16 &c) {
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bv), c, 0,
                                                 0, 0);
}

// Staging of MT*32 activation rows x 128 k: thread t moves chunk t%16 of rows
// t/16 + 16 i, i < 2*MT.
template <int MT>
struct Stage {
  const uint16_t *src[2 * MT];
  int off[2 * MT];
  uint4 v[2 * MT];
  __device__ void load(int ss) {
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) v[i] = *(const uint4 *)(src[i] + ss * 128);
  }
  __device__ void store(uint8_t *buf) {
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) *(uint4 *)(buf + off[i]) = v[i];
  }
};

// --------------------------------------------------------------------------- gate/up

template <int MT>
__device__ void gateup_item(const GemmArgs &a, uint8_t *lds, int e, int row0, int rows, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5;
  const int H = a.H, I = a.I, nss = H / 128;
  const QMat G = expert_mat(a.w0, a.s0, e, a.E, I, H);
  const QMat U = expert_mat(a.w1, a.s1, e, a.E, I, H);
  const int n = nb * kGateUpCols + wv * 32 + (lane & 31);
  const uint32_t *gq = G.q + (size_t)n * (H / 8) + hf * 8;
  const uint32_t *uq = U.q + (size_t)n * (H / 8) + hf * 8;
  const uint16_t *gs = G.s + (size_t)n * (H / 64) + hf;
  const uint16_t *gb = G.b + (size_t)n * (H / 64) + hf;
  const uint16_t *us = U.s + (size_t)n * (H / 64) + hf;
  const uint16_t *ub = U.b + (size_t)n * (H / 64) + hf;

  Stage<MT> st;
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i) {
    const int r = (tid >> 4) + 16 * i;
    const int tok = a.row_token[row0 + min(r, rows - 1)];
    st.src[i] = a.x + (size_t)tok * H + (tid & 15) * 8;
    st.off[i] = lds_off(r, tid & 15);
  }

  f32x16 accg[MT], accu[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    accg[t] = (f32x16){};
    accu[t] = (f32x16){};
  }

  st.load(0);
  uint4 g0 = *(const uint4 *)gq, g1 = *(const uint4 *)(gq + 4);
  uint4 u0 = *(const uint4 *)uq, u1 = *(const uint4 *)(uq + 4);
  float sg = fp16_to_f32(gs[0]), bg = fp16_to_f32(gb[0]);
  float su = fp16_to_f32(us[0]), bu = fp16_to_f32(ub[0]);
  st.store(lds);
  __syncthreads();

  for (int ss = 0; ss < nss; ++ss) {
    uint8_t *cur = lds + (ss & 1) * kBufBytes;
    const bool more = ss + 1 < nss;
    uint4 ng0, ng1, nu0, nu1;
    float nsg, nbg, nsu, nbu;
    if (more) {
      st.load(ss + 1);
      ng0 = *(const uint4 *)(gq + (ss + 1) * 16);
      ng1 = *(const uint4 *)(gq + (ss + 1) * 16 + 4);
      nu0 = *(const uint4 *)(uq + (ss + 1) * 16);
      nu1 = *(const uint4 *)(uq + (ss + 1) * 16 + 4);
      nsg = fp16_to_f32(gs[(ss + 1) * 2]);
      nbg = fp16_to_f32(gb[(ss + 1) * 2]);
      nsu = fp16_to_f32(us[(ss + 1) * 2]);
      nbu = fp16_to_f32(ub[(ss + 1) * 2]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t dg[4], du[4];
      dequant8_bf16(word_of(g0, g1, j), sg, bg, dg);
      dequant8_bf16(word_of(u0, u1, j), su, bu, du);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = t * 32 + (lane & 31);
        const u32x4 av = *(const u32x4 *)(cur + lds_off(row, hf * 8 + j));
        accg[t] = mfma(av, dg, accg[t]);
        accu[t] = mfma(av, du, accu[t]);
      }
    }
    if (more) {
      st.store(lds + ((ss + 1) & 1) * kBufBytes);
      g0 = ng0; g1 = ng1; u0 = nu0; u1 = nu1;
      sg = nsg; bg = nbg; su = nsu; bu = nbu;
    }
    __syncthreads();
  }

  // SwiGLU epilogue: h = silu(gate) * up, bf16
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = t * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
      if (r < rows) {
        const float gv = accg[t][v], uv = accu[t][v];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        a.h[(size_t)(row0 + r) * I + n] = f32_to_bf16(hv);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm_gateup(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];
  __shared__ int s_item;
  const int NB = a.I / kGateUpCols;
  const int n_items = a.ctrl->n_mblocks * NB;
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(a.queue, 1);
    __syncthreads();
    const int item = s_item;
    __syncthreads();
    if (item >= n_items) break;
    const int4 mb = a.mblocks[item / NB];
    const int nb = item % NB;
    switch (mb.w) {
      case 1: gateup_item<1>(a, lds, mb.x, mb.y, mb.z, nb); break;
      case 2: gateup_item<2>(a, lds, mb.x, mb.y, mb.z, nb); break;
      case 3: gateup_item<3>(a, lds, mb.x, mb.y, mb.z, nb); break;
      default: gateup_item<4>(a, lds, mb.x, mb.y, mb.z, nb); break;
    }
  }
}

// --------------------------------------------------------------------------- down

template <int MT>
__device__ void down_item(const GemmArgs &a, uint8_t *lds, int e, int row0, int rows, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5;
  const int H = a.H, I = a.I, nss = I / 128;
  const QMat D = expert_mat(a.w0, a.s0, e, a.E, H, I);
  const int n0 = nb * kDownCols + wv * 64 + (lane & 31);
  const int n1 = n0 + 32;
  const uint32_t *q0 = D.q + (size_t)n0 * (I / 8) + hf * 8;
  const uint32_t *q1 = D.q + (size_t)n1 * (I / 8) + hf * 8;
  const uint16_t *s0 = D.s + (size_t)n0 * (I / 64) + hf, *b0 = D.b + (size_t)n0 * (I / 64) + hf;
  const uint16_t *s1 = D.s + (size_t)n1 * (I / 64) + hf, *b1 = D.b + (size_t)n1 * (I / 64) + hf;

  Stage<MT> st;
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i) {
    const int r = (tid >> 4) + 16 * i;
    st.src[i] = a.x + (size_t)(row0 + min(r, rows - 1)) * I + (tid & 15) * 8;
    st.off[i] = lds_off(r, tid & 15);
  }

  f32x16 acc0[MT], acc1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc0[t] = (f32x16){};
    acc1[t] = (f32x16){};
  }

  st.load(0);
  uint4 w00 = *(const uint4 *)q0, w01 = *(const uint4 *)(q0 + 4);
  uint4 w10 = *(const uint4 *)q1, w11 = *(const uint4 *)(q1 + 4);
  float sa = fp16_to_f32(s0[0]), ba = fp16_to_f32(b0[0]);
  float sb = fp16_to_f32(s1[0]), bb = fp16_to_f32(b1[0]);
  st.store(lds);
  __syncthreads();

  for (int ss = 0; ss < nss; ++ss) {
    uint8_t *cur = lds + (ss & 1) * kBufBytes;
    const bool more = ss + 1 < nss;
    uint4 n00, n01, n10, n11;
    float nsa, nba, nsb, nbb;
    if (more) {
      st.load(ss + 1);
      n00 = *(const uint4 *)(q0 + (ss + 1) * 16);
      n01 = *(const uint4 *)(q0 + (ss + 1) * 16 + 4);
      n10 = *(const uint4 *)(q1 + (ss + 1) * 16);
      n11 = *(const uint4 *)(q1 + (ss + 1) * 16 + 4);
      nsa = fp16_to_f32(s0[(ss + 1) * 2]);
      nba = fp16_to_f32(b0[(ss + 1) * 2]);
      nsb = fp16_to_f32(s1[(ss + 1) * 2]);
      nbb = fp16_to_f32(b1[(ss + 1) * 2]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t d0[4], d1[4];
      dequant8_bf16(word_of(w00, w01, j), sa, ba, d0);
      dequant8_bf16(word_of(w10, w11, j), sb, bb, d1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = t * 32 + (lane & 31);
        const u32x4 av = *(const u32x4 *)(cur + lds_off(row, hf * 8 + j));
        acc0[t] = mfma(av, d0, acc0[t]);
        acc1[t] = mfma(av, d1, acc1[t]);
      }
    }
    if (more) {
      st.store(lds + ((ss + 1) & 1) * kBufBytes);
      w00 = n00; w01 = n01; w10 = n10; w11 = n11;
      sa = nsa; ba = nba; sb = nsb; bb = nbb;
    }
    __syncthreads();
  }

  // combine: out_acc[token] += gate * y (the shared expert's rows carry gate 1)
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = t * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
      if (r < rows) {
        const int tok = a.row_token[row0 + r];
        const float g = a.row_gate[row0 + r];
        float *o = a.out_acc + (size_t)tok * H;
        unsafeAtomicAdd(o + n0, g * acc0[t][v]);
        unsafeAtomicAdd(o + n1, g * acc1[t][v]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm_down(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];
  __shared__ int s_item;
  const int NB = a.H / kDownCols;
  const int n_items = a.ctrl->n_mblocks * NB;
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(a.queue, 1);
    __syncthreads();
    const int item = s_item;
    __syncthreads();
    if (item >= n_items) break;
    const int4 mb = a.mblocks[item / NB];
    const int nb = item % NB;
    switch (mb.w) {
      case 1: down_item<1>(a, lds, mb.x, mb.y, mb.z, nb); break;
      case 2: down_item<2>(a, lds, mb.x, mb.y, mb.z, nb); break;
      case 3: down_item<3>(a, lds, mb.x, mb.y, mb.z, nb); break;
      default: down_item<4>(a, lds, mb.x, mb.y, mb.z, nb); break;
    }
  }
}

// fp32 accumulator -> bf16 output, eight elements per thread
__global__ __launch_bounds__(256) void k_finalize(const float *acc, uint16_t *out, int64_t n8) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const float4 a0 = ((const float4 *)acc)[2 * i];
    const float4 a1 = ((const float4 *)acc)[2 * i + 1];
    uint4 o;
    o.x = pack_bf16x2(a0.x, a0.y);
    o.y = pack_bf16x2(a0.z, a0.w);
    o.z = pack_bf16x2(a1.x, a1.y);
    o.w = pack_bf16x2(a1.z, a1.w);
    ((uint4 *)out)[i] = o;
  }
}

}  // namespace

hipError_t launch_gemm_gateup(const GemmArgs &a, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_gateup, dim3(n_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs &a, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_down, dim3(n_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const float *acc, uint16_t *out, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  int64_t nb = (n8 + 255) / 256;
  if (nb > 4096) nb = 4096;
  if (nb < 1) nb = 1;
  hipLaunchKernelGGL(k_finalize, dim3((unsigned)nb), dim3(256), 0, s, acc, out, n8);
  return hipGetLastError();
}

}  // namespace moe
