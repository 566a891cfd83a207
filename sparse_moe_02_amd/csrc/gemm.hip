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
// MI355X mapping.  A work item is (M-block of one expert, N-block).  Eight waves split
// the N-block; each wave covers all rows of the M-block (1..4 tiles of 32), so a weight
// element is dequantised once per work item.  For a 128-wide K super-step, lane l of a
// wave owns weight row n = l%32 and the 64 consecutive k of half h = l/32: exactly eight
// packed words and one (scale, bias) pair.  Word j feeds MFMA j of the super-step, whose
// B operand wants 8 consecutive k per lane; the activation operand uses the same k
// assignment (k = 64h + 8j + i), so any k order inside the super-step is consistent.
// Every operand of a super-step -- activation rows (gathered by token for gate/up,
// contiguous h rows for down), packed weight words and scale/bias pairs -- goes from
// global memory straight to LDS (global_load_lds) into a two-stage ring, with 16-byte
// slots XOR-swizzled so the operand reads are free of bank conflicts.  The loads for
// super-step s+1 are in flight while s is multiplied; the loop holds no global load
// into registers, so the only memory wait is the explicit one at each step.
// Work items come from eight atomic queues, one per XCD: the N-blocks of one M-block
// run on the same XCD so its activation rows are fetched into one L2; an XCD whose
// queue is empty takes work from the others.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRowBytes = 256;                 // 128 bf16 per staged activation row
constexpr int kAStage = kBM * kRowBytes;       // 32 KiB: up to 128 activation rows
constexpr int kBSet = 256 * 64;                // 16 KiB: 256 weight rows x 64 B (128 codes)
constexpr int kSArr = 256 * 4;                 // 1 KiB: 256 rows x (2 fp16 of one array)
constexpr int kStageBytes = kAStage + 2 * kBSet + 4 * kSArr;  // 68 KiB

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));  // vmcnt(N), others free
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void g2l16(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void g2l4(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}

__device__ __forceinline__ QMat expert_mat(const QMat &routed, const QMat &shared, int e, int E, int N, int K) {
  if (e == E) return shared;
  QMat m;
  m.q = routed.q + (size_t)e * N * (K / 8);
  m.s = routed.s + (size_t)e * N * (K / 64);
  m.b = routed.b + (size_t)e * N * (K / 64);
  return m;
}

// activation tile: row r at r*256, 16-byte chunk c at slot c ^ (r & 15)
__device__ __forceinline__ int a_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 15)) << 4); }
// weight set: weight slot w (= 32*wave + lane%32) at w*64, 16-byte part p at p ^ ((w >> 2) & 3)
__device__ __forceinline__ int b_off(int slot, int part) { return slot * 64 + ((part ^ ((slot >> 2) & 3)) << 4); }

__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const uint32_t (&b)[4], const f32x16 &c) {
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bv), c, 0,
                                                 0, 0);
}

// One work item.  GU: gate/up + SwiGLU (K = H; weight set 0 = gate rows, set 1 = up rows,
// both row n of the lane).  Otherwise down + combine (K = I; sets 0/1 = rows n, n + 32).
template <int MT, bool GU>
__device__ void gemm_item(const GemmArgs &a, uint8_t *stage0, uint8_t *stage1, int *s_tok, float *s_gate, int e,
                          int row0, int rows, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5;
  const int H = a.H, I = a.I;
  const int K = GU ? H : I;
  const int N = GU ? I : H;  // rows of each weight matrix
  const int nss = K / 128;
  const QMat M0 = GU ? expert_mat(a.w0, a.s0, e, a.E, I, H) : expert_mat(a.w0, a.s0, e, a.E, H, I);
  const QMat M1 = GU ? expert_mat(a.w1, a.s1, e, a.E, I, H) : M0;
  // weight row of (set, slot): slot = 32*wave + j, j < 32
  auto wrow = [&](int set, int slot) {
    const int w = slot >> 5, j = slot & 31;
    const int n = GU ? nb * kGateUpCols + slot : nb * kDownCols + 64 * w + 32 * set + j;
    return min(n, N - 1);  // idle waves of a narrow layer load a valid row
  };
  const int n_lane = GU ? nb * kGateUpCols + 32 * wv + (lane & 31) : nb * kDownCols + 64 * wv + (lane & 31);
  const bool active = (GU ? nb * kGateUpCols + 32 * wv : nb * kDownCols + 64 * wv) < N;

  // --- this wave's share of each stage's loads: wave-uniform bases (scalar registers)
  // plus 32-bit per-lane byte offsets
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  // A: MT wave-loads of 1 KiB (4 rows), index i -> rows 4(wu + 8i) .. +3
  const char *abase = (const char *)a.x;
  uint32_t aoff[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = 4 * (wu + 8 * i) + (lane >> 4);
    const int rr = row0 + min(r, rows - 1);
    const uint32_t row_elem = GU ? (uint32_t)a.row_token[rr] * (uint32_t)H : (uint32_t)rr * (uint32_t)I;
    aoff[i] = 2u * (row_elem + 8u * (uint32_t)((lane & 15) ^ (r & 15)));
  }
  // B: 4 wave-loads of 1 KiB (16 weight slots), v = wu + 8i: set v/16, slots 16(v%16) ..
  const char *bbase[4];
  uint32_t boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = wu + 8 * i, set = v >> 4;
    const int slot = 16 * (v & 15) + (lane >> 2);
    bbase[i] = (const char *)(set ? M1.q : M0.q);
    boff[i] = 4u * ((uint32_t)wrow(set, slot) * (uint32_t)(K / 8) + 4u * (uint32_t)((lane & 3) ^ ((slot >> 2) & 3)));
  }
  // S: 2 wave-loads of 256 B (64 slots x 2 fp16), v = wu + 8i: array v/4 in
  // (scale set 0, bias set 0, scale set 1, bias set 1), slots 64(v%4) + lane
  const char *sbase[2];
  uint32_t soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = wu + 8 * i, arr = v >> 2, set = arr >> 1;
    const int slot = 64 * (v & 3) + lane;
    const QMat &M = set ? M1 : M0;
    sbase[i] = (const char *)((arr & 1) ? M.b : M.s);
    soff[i] = 2u * (uint32_t)wrow(set, slot) * (uint32_t)(K / 64);
  }
  auto issue = [&](int ss, uint8_t *st) {
#pragma unroll
    for (int i = 0; i < MT; ++i) g2l16(abase + aoff[i] + ss * 256, st + (wu + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) g2l16(bbase[i] + boff[i] + ss * 64, st + kAStage + (wu + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) g2l4(sbase[i] + soff[i] + ss * 4, st + kAStage + 2 * kBSet + (wu + 8 * i) * 256);
  };

  if (!GU && tid < MT * 32) {  // token and gate of every row, read back by the epilogue
    const int rr = row0 + min(tid, rows - 1);
    s_tok[tid] = a.row_token[rr];
    s_gate[tid] = a.row_gate[rr];
  }
  f32x16 acc0[MT], acc1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc0[t] = (f32x16){};
    acc1[t] = (f32x16){};
  }
  const int myslot = 32 * wv + (lane & 31);
  // multiply super-step ss from stage `st`
  auto compute = [&](const uint8_t *st) {
    const uint8_t *b0 = st + kAStage, *b1 = b0 + kBSet;
    const uint16_t *sp = (const uint16_t *)(b1 + kBSet);
    const float sa = fp16_to_f32(sp[myslot * 2 + hf]);
    const float ba = fp16_to_f32(sp[kSArr / 2 + myslot * 2 + hf]);
    const float sb = fp16_to_f32(sp[kSArr + myslot * 2 + hf]);
    const float bb = fp16_to_f32(sp[3 * kSArr / 2 + myslot * 2 + hf]);
    const uint4 w00 = *(const uint4 *)(b0 + b_off(myslot, 2 * hf));
    const uint4 w01 = *(const uint4 *)(b0 + b_off(myslot, 2 * hf + 1));
    const uint4 w10 = *(const uint4 *)(b1 + b_off(myslot, 2 * hf));
    const uint4 w11 = *(const uint4 *)(b1 + b_off(myslot, 2 * hf + 1));
    const uint32_t wa[8] = {w00.x, w00.y, w00.z, w00.w, w01.x, w01.y, w01.z, w01.w};
    const uint32_t wb[8] = {w10.x, w10.y, w10.z, w10.w, w11.x, w11.y, w11.z, w11.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t d0[4], d1[4];
      dequant8_bf16(wa[j], sa, ba, d0);
      dequant8_bf16(wb[j], sb, bb, d1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = t * 32 + (lane & 31);
        const u32x4 av = *(const u32x4 *)(st + a_off(row, hf * 8 + j));
        acc0[t] = mfma(av, d0, acc0[t]);
        acc1[t] = mfma(av, d1, acc1[t]);
      }
    }
  };
  // two-stage ring, unrolled by two so each read names one stage object and the
  // copies in flight name the other
  issue(0, stage0);
  for (int ss = 0; ss < nss; ss += 2) {
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();  // stage0 holds step ss for every wave; stage1 is free
    if (ss + 1 < nss) issue(ss + 1, stage1);
    if (active) compute(stage0);
    if (ss + 1 >= nss) break;
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();  // stage1 holds step ss+1; stage0 is free
    if (ss + 2 < nss) issue(ss + 2, stage0);
    if (active) compute(stage1);
  }
  // every wave is past its last LDS read before the next item refills the ring
  __builtin_amdgcn_s_barrier();
  if (!active) return;
  const int n0 = n_lane, n1 = n_lane + 32;

  if (GU) {
    // SwiGLU epilogue: h = silu(gate) * up, bf16
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = t * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (r < rows) {
          const float gv = acc0[t][v], uv = acc1[t][v];
          a.h[(size_t)(row0 + r) * I + n0] = f32_to_bf16(gv * sigmoid_fast(gv) * uv);
        }
      }
    }
  } else {
    // combine: out_acc[token] += gate * y (the shared expert's rows carry gate 1)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = t * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (r < rows) {
          const int tok = s_tok[r];
          const float g = s_gate[r];
          float *o = a.out_acc + (size_t)tok * H;
          unsafeAtomicAdd(o + n0, g * acc0[t][v]);
          unsafeAtomicAdd(o + n1, g * acc1[t][v]);
        }
      }
    }
  }
}

// Persistent grid.  Queue x serves M-blocks x, x+8, x+16, ... (all their N-blocks,
// consecutive); workgroup b starts on queue b % 8 (its XCD under round-robin
// dispatch) and moves on to the other queues when its own is empty.
template <bool GU>
__device__ void gemm_persistent(const GemmArgs &a) {
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStageBytes];
  __shared__ int s_tok[kBM];
  __shared__ float s_gate[kBM];
  __shared__ int s_item;
  const int NB = GU ? (a.I + kGateUpCols - 1) / kGateUpCols : (a.H + kDownCols - 1) / kDownCols;
  const int nmb = a.ctrl->n_mblocks;
  const int x0 = blockIdx.x % kXcds;
  for (int d = 0; d < kXcds; ++d) {
    const int x = (x0 + d) % kXcds;
    const int n_items = NB * ((nmb - x + kXcds - 1) / kXcds);
    for (;;) {
      if (threadIdx.x == 0) s_item = atomicAdd(&a.queue[x], 1);
      __syncthreads();
      const int item = s_item;
      __syncthreads();
      if (item >= n_items) break;
      const int4 mb = a.mblocks[x + kXcds * (item / NB)];
      const int nb = item % NB;
      switch (mb.w) {
        case 1: gemm_item<1, GU>(a, stage0, stage1, s_tok, s_gate, mb.x, mb.y, mb.z, nb); break;
        case 2: gemm_item<2, GU>(a, stage0, stage1, s_tok, s_gate, mb.x, mb.y, mb.z, nb); break;
        case 3: gemm_item<3, GU>(a, stage0, stage1, s_tok, s_gate, mb.x, mb.y, mb.z, nb); break;
        default: gemm_item<4, GU>(a, stage0, stage1, s_tok, s_gate, mb.x, mb.y, mb.z, nb); break;
      }
    }
  }
}

__global__ __launch_bounds__(kGemmThreads) void k_gemm_gateup(GemmArgs a) { gemm_persistent<true>(a); }
__global__ __launch_bounds__(kGemmThreads) void k_gemm_down(GemmArgs a) { gemm_persistent<false>(a); }

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
  hipLaunchKernelGGL(k_gemm_gateup, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs &a, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_down, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
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
