// Measured ceilings for the MoE layer's kernels on the current GPU (not part of the layer:
// the benchmark times these beside it).
//
// "Optimizing on-device inference for Apple Silicon", section "Limits of further
// optimization": each kernel's efficiency is stated against the fastest sustained
// weight-read rate for its access pattern and against the matrix units' peak, and the
// sparse GEMV is re-run with its arithmetic removed to show that weight reads bound it.
// The probes here give the same reference points on an MI355X:
//   probe_read_stream   -- a plain read of a large buffer with 16-byte loads (HBM read
//                          ceiling);
//   probe_mfma          -- a register-only loop of v_mfma_f32_32x32x16_bf16 (the matrix
//                          units' sustained rate, clock included);
//   probe_mfma_data     -- the same loop on operands loaded from memory (random bf16 data
//                          in the benchmark: the matrix units' rate on real bits, which
//                          draw more power than the constant operands above), ten
//                          accumulators, two waves per SIMD;
//   probe_dequant_mfma  -- the grouped GEMM's register pipeline without LDS: per 16-k
//                          slice two packed words dequantised (the library's own int4 ->
//                          bf16 routine) and 2 x 5 MFMAs, in the kernel's issue pattern
//                          (the ceiling of dequantising inside the MFMA loop);
//   probe_empty         -- an empty kernel (launch cost, e.g. replayed from a HIP graph);
//   probe_expert_stream -- the nine active experts' packed weights of one decode step
//                          (gate, up, down codes + fp16 scale/bias, 16-byte loads), read
//                          in one phase with the experts already known: with the dequant
//                          dot products of the decode GEMVs (arith = 1) or with the
//                          arithmetic replaced by an XOR of the loaded words (arith = 0).
// Every kernel writes its result to a sink only under a condition the data never meets,
// so the loads and the arithmetic cannot be dropped by the compiler.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../csrc/common.hpp"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(256) void k_read_stream(const uint4 *__restrict__ buf, size_t n16,
                                                      uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Four independent accumulation chains per wave (the MFMA's latency is covered by the
// other chains and by the other waves of the SIMD).
__global__ __launch_bounds__(256) void k_mfma(int iters, float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const u32x4 av = {0x3f803f80u + lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const u32x4 bv = {0x3c003c00u, 0x3c003c00u + lane, 0x3c003c00u, 0x3c003c00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, av), b = __builtin_bit_cast(bf16x8, bv);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (s == -1.0f) sink[blockIdx.x] = s;
}

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4p;

// operands from memory: 5 activation-like and 2 weight-like fragments per lane
__global__ __launch_bounds__(512) void k_mfma_data(const u32x4p *__restrict__ src, int iters,
                                                    float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  u32x4p a[5], b[2];
#pragma unroll
  for (int i = 0; i < 5; ++i) a[i] = src[(blockIdx.x * 8 + i) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = src[(blockIdx.x * 8 + 5 + i) * 64 + lane];
  f32x16 c[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) c[i] = (f32x16){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 10; ++i)
      c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[i & 1]),
                                                     __builtin_bit_cast(bf16x8, a[i % 5]), c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 10; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  if (s == -1.2345f) sink[blockIdx.x] = s;
}

// one 128-k super-step's worth of the grouped GEMM's registers, repeated: 8 slices, each
// with the two tiles' words dequantised and 2 x 5 MFMAs (5 row tiles)
__global__ __launch_bounds__(512) void k_dequant_mfma(const u32x4p *__restrict__ src, int iters,
                                                       float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  u32x4p a[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) a[i] = src[(blockIdx.x * 8 + i) * 64 + lane];
  const u32x4p wsrc = src[(blockIdx.x * 8 + 6) * 64 + lane];
  uint32_t w0 = wsrc[0], w1 = wsrc[1];
  const moe::DeqPair dp = moe::deq_pair(0.01f + lane * 1e-4f, -0.08f);
  f32x16 acc[5][2];
#pragma unroll
  for (int t = 0; t < 5; ++t) acc[t][0] = acc[t][1] = (f32x16){};
  uint32_t d0[4], d1[4];
  moe::dequant8_bf16_m(w0, dp, d0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      moe::dequant8_bf16_m(w1, dp, d1);
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        const u32x4p wv = {d0[0], d0[1], d0[2], d0[3]};
        acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv),
                                                            __builtin_bit_cast(bf16x8, a[t]), acc[t][0], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      w0 = (w0 >> 3) | (w0 << 29);
      w1 = (w1 >> 5) | (w1 << 27);
      moe::dequant8_bf16_m(w0, dp, d0);
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        const u32x4p wv = {d1[0], d1[1], d1[2], d1[3]};
        acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv),
                                                            __builtin_bit_cast(bf16x8, a[t]), acc[t][1], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 5; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[t][0][j] + acc[t][1][j];
  if (s == -1.2345f) sink[blockIdx.x] = s;
}

__global__ void k_empty() {}

struct Mat {
  const uint32_t *q;   // codes in 16-row x 128-k tiles
  const uint16_t *s;   // fp16 scale, 16-row tiles
  const uint16_t *b;   // fp16 bias
};
struct ExpertStreamArgs {
  Mat gate[9], up[9], down[9];  // the nine active experts (slot 8: the shared one)
  const uint16_t *x;            // bf16 [H]
  int H, I, n_slots;
  float *sink;
};

__device__ __forceinline__ size_t code_index(size_t n, int w, int K) {
  return ((n >> 4) * (size_t)(K / 128) + (size_t)(w >> 4)) * 256u + (n & 15u) * 16u + (size_t)(w & 15);
}
__device__ __forceinline__ size_t qp_index(size_t n, int g, int G) {
  return ((n / 16) * (size_t)G + (size_t)g) * 16 + (n % 16);
}
__device__ __forceinline__ float f16(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// sum_i v_i q_i over the 32 codes of a 16-byte piece
__device__ __forceinline__ float dot32(const uint4 &w, const float *v) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) s = __builtin_fmaf(v[8 * q + j], (float)((ws[q] >> (4 * j)) & 0xfu), s);
  return s;
}

// Unit u of the stream: u < n_slots*I: gate and up row u%I of slot u/I (K = H);
// otherwise down row n = u - n_slots*I of every slot (K = I).  One wave per unit, a lane
// per 32-element chunk (16-byte code loads), chunks c = lane + 64 p.
template <bool ARITH>
__global__ __launch_bounds__(256) void k_expert_stream(ExpertStreamArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), nwaves = gridDim.x * 4;
  const int H = a.H, I = a.I, S = a.n_slots;
  const int n_units = S * I + H;
  float facc = 0.f;
  uint32_t xacc = 0;
  for (int u = wave; u < n_units; u += nwaves) {
    if (u < S * I) {
      const int j = u / I, r = u - j * I;
      for (int c = lane; c < H / 32; c += 64) {
        const uint4 g = *(const uint4 *)(a.gate[j].q + code_index(r, 4 * c, H));
        const uint4 w = *(const uint4 *)(a.up[j].q + code_index(r, 4 * c, H));
        const size_t qi = qp_index(r, c / 2, H / 64);
        const uint16_t gs = a.gate[j].s[qi], gb = a.gate[j].b[qi], us = a.up[j].s[qi], ub = a.up[j].b[qi];
        if (ARITH) {
          float v[32], xs = 0.f;
          const uint4 *xp = (const uint4 *)(a.x + 32 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 xv = xp[q];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[8 * q + 2 * i] = bf((uint16_t)xw[i]);
              v[8 * q + 2 * i + 1] = bf((uint16_t)(xw[i] >> 16));
            }
          }
#pragma unroll
          for (int i = 0; i < 32; ++i) xs += v[i];
          facc += f16(gs) * dot32(g, v) + f16(gb) * xs + f16(us) * dot32(w, v) + f16(ub) * xs;
        } else {
          xacc ^= g.x ^ g.y ^ g.z ^ g.w ^ w.x ^ w.y ^ w.z ^ w.w ^ gs ^ gb ^ us ^ ub;
        }
      }
    } else {
      const int n = u - S * I;
      for (int j = 0; j < S; ++j)
        for (int c = lane; c < I / 32; c += 64) {
          const uint4 d = *(const uint4 *)(a.down[j].q + code_index(n, 4 * c, I));
          const size_t qi = qp_index(n, c / 2, I / 64);
          const uint16_t ds = a.down[j].s[qi], db = a.down[j].b[qi];
          if (ARITH) {
            float v[32], vs = 0.f;
            const uint4 *xp = (const uint4 *)(a.x + 32 * c);  // stands in for h
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint4 xv = xp[q];
              const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                v[8 * q + 2 * i] = bf((uint16_t)xw[i]);
                v[8 * q + 2 * i + 1] = bf((uint16_t)(xw[i] >> 16));
              }
            }
#pragma unroll
            for (int i = 0; i < 32; ++i) vs += v[i];
            facc += f16(ds) * dot32(d, v) + f16(db) * vs;
          } else {
            xacc ^= d.x ^ d.y ^ d.z ^ d.w ^ ds ^ db;
          }
        }
    }
  }
  if (ARITH ? (facc == -1.0f) : (xacc == 0x9e3779b9u)) a.sink[blockIdx.x] = facc + (float)xacc;
}

// The same bytes as one flat read: n_seg device arrays (the nine experts' matrices and
// the router), 16 KB per workgroup (256 threads x 4 loads of 16 bytes in flight), each
// workgroup inside one segment.  table: the segments' base addresses, their sizes in
// 16-byte units, and the index of each segment's first workgroup (n_seg+1 entries).
__global__ __launch_bounds__(256) void k_flat_stream(const uint64_t *table, int n_seg, uint32_t *sink) {
  const uint64_t *base = table, *n16 = table + 128, *wg0 = table + 256;
  int lo = 0, hi = n_seg - 1;  // last segment whose first workgroup <= blockIdx.x
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (wg0[mid] <= blockIdx.x) lo = mid; else hi = mid - 1;
  }
  const uint4 *p = (const uint4 *)base[lo];
  const size_t n = n16[lo], i0 = (size_t)(blockIdx.x - wg0[lo]) * 1024 + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = i0 + 256 * u < n ? p[i0 + 256 * u] : make_uint4(0, 0, 0, 0);
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// One ticket per workgroup on completion counters, as a launch's last-arriver detection
// does: mode 0, every workgroup on one counter; mode 1, eight counters (workgroup b on
// counter 1 + b%8), the last of each then on counter 0.  The last arriver resets what it
// used, so the counters are zero between launches.
__global__ __launch_bounds__(256) void k_ticket(int *ctr, int mode, int stride) {
  if (threadIdx.x != 0) return;
  const int G = gridDim.x, b = blockIdx.x;
  if (mode == 0) {
    if (__hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1)
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int g = b % 8, n_g = G / 8 + (g < G % 8 ? 1 : 0);
  int *c = ctr + stride * (1 + g);
  if (__hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_g - 1) {
    __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == min(G, 8) - 1)
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Hand-off latency between workgroups.  Workgroup b < 8 stores an 8-byte record {value,
// tag} to slot[b]; every other workgroup b polls slot[(b + shift) % 8] until the tag is
// this launch's (at most `spins` polls) and records, in the device's 100 MHz clock, when
// it saw it.  mode 0: agent-scope relaxed atomic store and loads (coherent across XCDs);
// mode 1: a plain store, and loads that first invalidate the CU's vector cache and then
// read through it (coherent only through the L2 the two workgroups share).  Under the
// round-robin placement of workgroups on XCDs, shift 0 pairs workgroups on the same XCD.
// out[b] = {clock at the store (producers) or at the sighting, clock at start, polls, XCD}.
__device__ __forceinline__ uint64_t ld_inv_l2(const uint64_t *p) {
  uint64_t v;
  asm volatile("buffer_inv sc0\n\tglobal_load_dwordx2 %0, %1, off sc0\n\ts_waitcnt vmcnt(0)"
               : "=v"(v)
               : "v"(p)
               : "memory");
  return v;
}

__global__ __launch_bounds__(64) void k_handoff(uint64_t *slot, uint32_t tag, int mode, int shift, int spins,
                                                 uint64_t *out) {
  if (threadIdx.x != 0) return;
  const int b = blockIdx.x;
  const uint64_t t_start = wall_clock64();
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xfu;  // HW_REG_XCC_ID[3:0]
  uint64_t t = 0, polls = 0;
  if (b < 8) {
    const uint64_t rec = ((uint64_t)tag << 32) | (uint32_t)b;
    if (mode == 0) {
      __hip_atomic_store(slot + b, rec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      slot[b] = rec;
    }
    __builtin_amdgcn_s_waitcnt(0);
    t = wall_clock64();
  } else {
    const uint64_t *p = slot + (b + shift) % 8;
    for (; polls < (uint64_t)spins; ++polls) {
      const uint64_t r = mode == 0 ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ld_inv_l2(p);
      if ((uint32_t)(r >> 32) == tag) break;
    }
    t = wall_clock64();
  }
  out[4 * b + 0] = t;
  out[4 * b + 1] = t_start;
  out[4 * b + 2] = polls;
  out[4 * b + 3] = xcc;
}

}  // namespace

extern "C" {

// table: device array of 384 words (base addresses, sizes in 16-byte units, first
// workgroup of each segment; n <= 127); grid: the total workgroups (table[256 + n]).
int probe_flat_stream(const void *table, int n, void *sink, int grid, hipStream_t s) {
  if (n < 1 || n > 127 || grid < 1) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_flat_stream, dim3(grid), dim3(256), 0, s, (const uint64_t *)table, n, (uint32_t *)sink);
  return (int)hipGetLastError();
}

// ctr: 9 * stride ints, zero before the first launch.
int probe_ticket(void *ctr, int mode, int stride, int grid, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_ticket, dim3(grid), dim3(256), 0, s, (int *)ctr, mode, stride);
  return (int)hipGetLastError();
}

// slot: 8 words; out: 4*grid words; grid > 8.
int probe_handoff(void *slot, uint32_t tag, int mode, int shift, int spins, void *out, int grid, hipStream_t s) {
  if (grid <= 8 || spins < 1) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_handoff, dim3(grid), dim3(64), 0, s, (uint64_t *)slot, tag, mode, shift, spins,
                     (uint64_t *)out);
  return (int)hipGetLastError();
}

// All pointers are device pointers; sink holds at least `grid` words.  Return a HIP
// error code (0 = launched).
int probe_read_stream(const void *buf, size_t bytes, void *sink, int grid, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_read_stream, dim3(grid), dim3(256), 0, s, (const uint4 *)buf, bytes / 16, (uint32_t *)sink);
  return (int)hipGetLastError();
}

int probe_mfma(int iters, void *sink, int grid, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_mfma, dim3(grid), dim3(256), 0, s, iters, (float *)sink);
  return (int)hipGetLastError();
}

// src: grid * 8 * 64 16-byte values (the fragments each workgroup's waves read).
int probe_mfma_data(const void *src, int iters, void *sink, int grid, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_mfma_data, dim3(grid), dim3(512), 0, s, (const u32x4p *)src, iters, (float *)sink);
  return (int)hipGetLastError();
}

int probe_dequant_mfma(const void *src, int iters, void *sink, int grid, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_dequant_mfma, dim3(grid), dim3(512), 0, s, (const u32x4p *)src, iters, (float *)sink);
  return (int)hipGetLastError();
}

int probe_empty(int grid, int threads, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_empty, dim3(grid), dim3(threads), 0, s);
  return (int)hipGetLastError();
}

// mats: host array of 9 x 3 x 3 device pointers, [slot][gate, up, down][q, scale, bias],
// in the layouts of include/moe.h (gate/up [I][H], down [H][I] per slot).
int probe_expert_stream(const void *const *mats, const void *x, int H, int I, int arith, void *sink, int grid,
                        hipStream_t s) {
  // x [H] also stands in for the down projection's input, so I <= H; rows in 16-row tiles
  if (I > H || H % 128 || I % 128 || grid < 1) return (int)hipErrorInvalidValue;
  ExpertStreamArgs a{};
  for (int j = 0; j < 9; ++j) {
    Mat *m[3] = {&a.gate[j], &a.up[j], &a.down[j]};
    for (int t = 0; t < 3; ++t) {
      m[t]->q = (const uint32_t *)mats[(j * 3 + t) * 3 + 0];
      m[t]->s = (const uint16_t *)mats[(j * 3 + t) * 3 + 1];
      m[t]->b = (const uint16_t *)mats[(j * 3 + t) * 3 + 2];
    }
  }
  a.x = (const uint16_t *)x;
  a.H = H;
  a.I = I;
  a.n_slots = 9;
  a.sink = (float *)sink;
  (void)hipGetLastError();
  if (arith)
    hipLaunchKernelGGL(k_expert_stream<true>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_expert_stream<false>, dim3(grid), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

}  // extern "C"
