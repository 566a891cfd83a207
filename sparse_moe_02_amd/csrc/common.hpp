// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 1/(1+exp(-a)) with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float sigmoid_fast(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// Round to nearest even, packing (lo, hi) into one word (compiles to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

// c + a.lo b.lo + a.hi b.hi for two pairs of bf16 (v_dot2_f32_bf16; the products are exact
// in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Codes p and p + 4 (p < 4) of a packed word of eight 4-bit codes as the bf16 pair
// (128 + code p, 128 + code p + 4): each code lands in the low mantissa bits of 128
// (0x4300), so the numbers are exact.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int p) {
  return ((w >> (4 * p)) & 0x000f000fu) | 0x43004300u;
}

// Eight bf16 values v0..v7 held as natural pairs (v0,v1) (v2,v3) (v4,v5) (v6,v7), regrouped
// into the pairs (v_p, v_p+4) that match code_pair.
__device__ __forceinline__ void pairs_p4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t *o) {
  o[0] = __builtin_amdgcn_perm(w2, w0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(w2, w0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(w3, w1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(w3, w1, 0x07060302u);
}

__device__ __forceinline__ float fp16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// A scale or bias value: fp16 bits, or bf16 bits when bf16 (the pages' checkpoint format).
__device__ __forceinline__ float qp_f32(uint32_t v, bool bf16) {
  return bf16 ? __uint_as_float((v & 0xffffu) << 16) : fp16_to_f32((uint16_t)v);
}

// Scale and bias arrays (G groups of 64 per row) are stored in tiles of kQpRows rows:
// the tile's values of one group are contiguous, groups follow each other.
constexpr int kQpRows = 16;
// Code words are stored in tiles of 16 rows x 128 k (16 words per row per tile): word w
// of row n (K/8 words per row) is at code_index(n, w, K).
__device__ __forceinline__ size_t code_index(size_t n, int w, int K) {
  return ((n >> 4) * (size_t)(K / 128) + (size_t)(w >> 4)) * 256u + (n & 15u) * 16u + (size_t)(w & 15);
}
__device__ __forceinline__ size_t qp_index(size_t n, int g, int G) {
  return ((n / kQpRows) * (size_t)G + (size_t)g) * kQpRows + (n % kQpRows);
}

// Dequantise the 8 codes of one packed word with one (scale, bias) and pack the eight
// weights to 4 bf16x2 words (element order k, k+1, ... low half first): w = s*code + b
// in fp32, then rounded to nearest even.  The int4 -> float step is the fp16 "magic
// number" conversion published by Kim et al., "Who Says Elephants Can't Run: Bringing
// Large Scale MoE Models into Cloud Scale Production" (arXiv 2211.10017): OR-ing a 4-bit
// code into the mantissa of the fp16 number 1024 gives exactly 1024 + code.  Here, for
// each code pair (2j, 2j+1), one byte permute and one and-or build a dword whose low
// half is the fp16 1024 + c_2j and whose high half is the fp16 1024 + 16 c_2j+1 (both
// exact), and a mixed-precision fma maps each half to s c + b in fp32: the low half
// with (s, b - 1024 s), the high half with (s/16, b - 64 s) -- the DeqPair below.  20
// VALU instructions per word.
struct DeqPair {
  float s_lo, b_lo, s_hi, b_hi;
  uint32_t nib;  // 0x00f0000f held in a vector register, so the mask-and-or is one v_and_or_b32
};
__device__ __forceinline__ DeqPair deq_pair(float s, float b) {
  uint32_t nib;
  asm("v_mov_b32 %0, 0x00f0000f" : "=v"(nib));
  return DeqPair{s, __builtin_fmaf(-1024.0f, s, b), 0.0625f * s, __builtin_fmaf(-64.0f, s, b), nib};
}
__device__ __forceinline__ void dequant8_bf16_m(uint32_t w, const DeqPair &p, uint32_t out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte j of w to bytes 0 and 2 (selector bytes j, j+4 of the {w, w} pair)
    const uint32_t sel = (uint32_t)j | ((uint32_t)j << 16) | 0x0c000c00u;
    const uint32_t x = (__builtin_amdgcn_perm(w, w, sel) & p.nib) | 0x64006400u;
    const float lo = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu)), p.s_lo, p.b_lo);
    const float hi = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16)), p.s_hi, p.b_hi);
    out[j] = pack_bf16x2(lo, hi);
  }
}

// ---------------------------------------------------------------- direct-to-LDS loads

// 16 bytes per lane from gbase + voff into LDS: lane i's bytes land at lds + 16 i (lds is
// wave-uniform).  Issued from inline asm so the compiler neither waits for it nor orders
// LDS reads behind it on its own: the caller counts its loads, waits with vm_wait_dyn and
// publishes the data with a barrier.
// gbase must be wave-uniform; it is read from the first lane, so the compiler keeps it in
// scalar registers even where it cannot prove the uniformity itself.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(uniform_ptr(gbase))
               : "memory", "m0");
}

// The same with 4 bytes per lane (lane i's bytes land at lds + 4 i).
__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(uniform_ptr(gbase))
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

template <int N>
__device__ __forceinline__ void vm_wait_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(m) for the largest m <= n of a small ladder (n: loads that may stay in
// flight; a smaller count only waits longer).
__device__ __forceinline__ void vm_wait_dyn(int n) {
  if (n >= 16) {
    if (n >= 32) vm_wait_n<32>(); else if (n >= 24) vm_wait_n<24>(); else vm_wait_n<16>();
  } else if (n >= 8) {
    if (n >= 12) vm_wait_n<12>(); else if (n >= 10) vm_wait_n<10>(); else vm_wait_n<8>();
  } else if (n >= 4) {
    if (n >= 6) { if (n >= 7) vm_wait_n<7>(); else vm_wait_n<6>(); } else { if (n >= 5) vm_wait_n<5>(); else vm_wait_n<4>(); }
  } else {
    if (n >= 2) { if (n >= 3) vm_wait_n<3>(); else vm_wait_n<2>(); } else { if (n >= 1) vm_wait_n<1>(); else vm_wait_n<0>(); }
  }
}

// ---------------------------------------------------------------- wave reductions

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND = false>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, BOUND));
}

// Sum over the 16 lanes of each DPP row; every lane of the row receives the row sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return v;
}

// Maximum over the 16 lanes of each DPP row, broadcast to the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return v;
}

// Wave reductions read back from lane 63, so every lane gets the same (uniform) value:
// DPP steps within each row of 16 lanes (every lane of a row ends with its row's result),
// then the row broadcasts 15 and 31 fold rows 0..2 into row 3 -- six DPP steps and one
// v_readlane, no LDS round trip.  Called by whole waves only.

// 64-bit DPP move: lanes of rows outside ROW_MASK get `old`.
template <int C, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_d(double x, double old = 0.0) {
  const uint64_t b = (uint64_t)__double_as_longlong(x), o = (uint64_t)__double_as_longlong(old);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)b, C, ROW_MASK, 0xf, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32), (int)(uint32_t)(b >> 32), C, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xa, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Binary64 sum: six levels of additions on the path of every lane's value.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_d<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_d<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_d<0x124>(v);       // row_ror:4
  v += dpp_d<0x128>(v);       // row_ror:8
  v += dpp_d<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_d<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return readlane_d(v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the wave's lanes: DPP row shifts by 1, 2, 4 and 8 within each
// 16-lane row (lanes shifted in from outside the row read 0), then the row broadcasts 15 and
// 31 carry the earlier rows' totals forward.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

// wave minimum of mn and maximum of mx together
__device__ __forceinline__ void wave_minmax_f64(double &mn, double &mx) {
  mn = fmin(mn, dpp_d<0xB1>(mn)); mx = fmax(mx, dpp_d<0xB1>(mx));
  mn = fmin(mn, dpp_d<0x4E>(mn)); mx = fmax(mx, dpp_d<0x4E>(mx));
  mn = fmin(mn, dpp_d<0x124>(mn)); mx = fmax(mx, dpp_d<0x124>(mx));
  mn = fmin(mn, dpp_d<0x128>(mn)); mx = fmax(mx, dpp_d<0x128>(mx));
  mn = fmin(mn, dpp_d<0x142, 0xa>(mn, mn)); mx = fmax(mx, dpp_d<0x142, 0xa>(mx, mx));
  mn = fmin(mn, dpp_d<0x143, 0xc>(mn, mn)); mx = fmax(mx, dpp_d<0x143, 0xc>(mx, mx));
  mn = readlane_d(mn, 63);
  mx = readlane_d(mx, 63);
}

// Cross-workgroup hand-off without cache maintenance: agent-scope relaxed atomic
// stores/loads are coherent across XCDs; draining vmcnt after the data stores orders
// them before a following relaxed ticket update.
template <class T>
__device__ __forceinline__ void st_agent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_agent(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This lane's index in its wave (v_mbcnt over all lanes), computed where it is used: the
// volatile asm keeps the compiler from computing it once at the start and holding it in a
// register (or spilling it) through the code in between.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0xF70); }  // vmcnt(0)
__device__ __forceinline__ int ticket(int *p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tag of this call's hand-off records, taken at the start of the call with no work at its
// end.  Eight call counters (64-bit, 256 bytes apart): workgroup b adds to counter b % 8,
// 1 each except the first workgroup of every group, which adds the rest of kEpochUnit
// (workgroup 0 also adds a whole unit to the counters of groups with no workgroup), so
// every call moves every counter by exactly kEpochUnit and each ticket of the n-th call
// on a workspace lies in [n kEpochUnit, (n+1) kEpochUnit) whatever the grid, for both
// decode kernels.  Calls on one stream run one after the other, so no call's tickets mix
// with the next one's.  The tag is n mod (2^32 - 1) plus 1: never 0 (the value of
// cleared records) and different in consecutive calls.
constexpr uint64_t kEpochUnit = uint64_t(1) << 24;
// The ticket (the atomic's return value is waited for at its first use) ...  The
// counter's address carries a per-lane zero the compiler cannot see through: with a
// uniform address it would combine the active lanes' adds into one and broadcast the
// result, which waits for the atomic's round trip right where it is issued.
__device__ __forceinline__ uint64_t epoch_ticket(uint64_t *ctr, int stride_u64, int b, int G) {
  const int g = b & 7;
  const int n_g = G / 8 + (g < G % 8 ? 1 : 0);
  if (b == 0)
    for (int g2 = G; g2 < 8; ++g2)
      __hip_atomic_fetch_add(ctr + (size_t)g2 * stride_u64, kEpochUnit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t w = b < 8 ? kEpochUnit - (uint64_t)(n_g - 1) : uint64_t(1);
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return __hip_atomic_fetch_add(ctr + (size_t)g * stride_u64 + z, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// ... and the tag it gives.
__device__ __forceinline__ uint64_t lane0_u64(uint64_t v) {
  return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         __builtin_amdgcn_readfirstlane((uint32_t)v);
}
__device__ __forceinline__ uint32_t epoch_of(uint64_t t) { return (uint32_t)((t / kEpochUnit) % 0xffffffffull) + 1u; }

}  // namespace moe
