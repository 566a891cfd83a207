// Grouped GEMMs of the prefill form, bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation and int4 weights dequantised on chip.
//
// "Optimizing on-device inference for Apple Silicon", section "Prefill > Dequantize
// weights during matmul": the grouped GEMM reconstructs one small weight tile at a time
// in on-chip memory and multiplies it with the routed activation rows, accumulating in
// fp32; the expanded weight array never exists in memory.  Section "Decode > Reduce
// intermediate and state traffic" fuses the gated activation with the input
// projections and the routing score and shared expert with the output projection; the
// same fusions are applied here: SwiGLU in the gate/up epilogue, the routing weight in
// the down epilogue (the k+1 rows of a token are summed by a short gather kernel).
//
// MI355X mapping.  A work item is (M-block of one expert, N-block).  Eight waves (two
// per SIMD) split the N-block; each wave covers all rows of the M-block (1..5 tiles of
// 32), so a weight element is dequantised once per work item, and each wave interleaves
// its dequant VALU work between its own MFMAs (k-slice software pipeline).  For a 128-wide K super-step, lane l of a
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
// run on the same XCD so its activation rows are fetched into one L2; a workgroup whose
// queue is empty reads all eight counts in one round trip and takes work from the
// fullest.  When the last round of gate/up items would leave most of the grid idle, its
// items are split along K into pieces whose partial sums are combined by the piece that
// finishes last.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRowBytes = 256;                 // 128 bf16 per staged activation row
constexpr int kAStage = kBM * kRowBytes;       // 40 KiB: up to 160 activation rows
constexpr int kBStage = 512 * 64;              // 32 KiB: 512 weight rows x 64 B (128 codes)
constexpr int kSStage = 2 * 512 * 4;           // 4 KiB: scales then biases, 2 groups per row
constexpr int kStageBytes = kAStage + kBStage + kSStage;  // 76 KiB

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));  // vmcnt(N), others free
}

__device__ __forceinline__ QMat expert_mat(const QMat &routed, const QMat &shared, int e, int E, int N, int K) {
  if (e == E) return shared;
  QMat m;
  m.q = routed.q + (size_t)e * N * (K / 8);
  m.s = routed.s + (size_t)e * N * (K / 64);
  m.b = routed.b + (size_t)e * N * (K / 64);
  return m;
}

// activation tile: row r at r*256, 16-byte chunk c at slot c ^ (r & 15) (the stage loads
// place the chunks so, and the fragment reads below undo it)
// weights: slot w (one weight row) at w*64, 16-byte part p at p ^ ((w >> 2) & 3)
__device__ __forceinline__ int b_off(int slot, int part) { return slot * 64 + ((part ^ ((slot >> 2) & 3)) << 4); }

// D += W X^T for a 32x32 tile: the weights are the row operand and the activations the
// column operand, so lane l holds token row l%32 of the tile and output columns
// 8q + 4(l/32) + {0,1,2,3} in accumulator entries 4q..4q+3 (four consecutive columns).
__device__ __forceinline__ f32x16 mfma(const uint32_t (&w)[4], const u32x4 &x, const f32x16 &c) {
  const u32x4 wv = {w[0], w[1], w[2], w[3]};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, x), c, 0,
                                                 0, 0);
}

// One work item, eight waves (two per SIMD).  Each wave owns two 32-column MFMA tiles of
// weight rows: GU (gate/up + SwiGLU, K = H): tile 0 = gate row n, tile 1 = up row n with
// n = nb*256 + 32*wave + lane%32; down (K = I): tile i = row nb*512 + 64*wave + 32 i +
// lane%32.  Weight slot (0..511) = 64*wave + 32*tile + lane%32.
// A split gate/up item: this launch computes K-steps [ks0, ks1) of it as piece p of S.
// Every piece stores its fp32 partial sums in its slot of `slots` (device-scope stores)
// and takes a ticket; the piece that takes the last ticket reads back the S partial sums
// and adds them in piece order, so the result does not depend on which piece finishes
// last, and runs the epilogue.  No piece waits for another.
struct Piece {
  int ti;  // split item: slots [ti*S, ti*S + S) of GemmArgs::part, ticket ti; -1: whole item
  int S, p;
};

// `claim` (wave-uniform; null: none) is the queue counter the next work item will be
// taken from: wave 0 takes the ticket once the item's last multiply is done, so the
// atomic's round trip overlaps the epilogue, and leaves the value in *s_pend when the
// item ends.
// W16: the weights are bf16 matrices (MOE_F_SEPARATE_DEQUANT: expanded by k_dequant_w16
// in 16-row x 32-k tiles of 1 KB), a super-step is 32 k (two MFMA slices; each weight
// row's 64 bytes per step land in the same B layout as the packed codes), and there is
// no scale/bias stage and no dequantisation.
template <int MT, bool GU, bool W16>
__device__ void gemm_item(const GemmArgs &a, uint8_t *stage0, uint8_t *stage1, float *s_gate, int *s_last, int e,
                          int row0, int rows, int nb, int ks0, int ks1, const Piece &pc, int *claim, int *s_pend,
                          int wv0) {
  // thread index made opaque so per-lane address arithmetic is computed per item instead
  // of being hoisted out of the persistent loop (where every row-tile variant's copy
  // would hold registers for the whole kernel)
  int tid = (wv0 << 6) + lane_now();
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I;
  const int K = GU ? H : I;
  const int N = GU ? I : H;  // rows of each weight matrix
  constexpr int KF = W16 ? 4 : 1;  // the bf16 tiles are laid out as packed codes of a 4x longer row
  const QMat M0 = GU ? expert_mat(a.w0, a.s0, e, a.E, I, KF * H) : expert_mat(a.w0, a.s0, e, a.E, H, KF * I);
  const QMat M1 = GU ? expert_mat(a.w1, a.s1, e, a.E, I, KF * H) : M0;
  auto slot_mat = [&](int slot) -> const QMat & { return (GU && ((slot >> 5) & 1)) ? M1 : M0; };
  auto slot_row = [&](int slot) {
    const int w = slot >> 6, t = (slot >> 5) & 1, j = slot & 31;
    const int n = GU ? nb * kGateUpCols + 32 * w + j : nb * kDownCols + 64 * w + 32 * t + j;
    return min(n, N - 1);  // idle waves of a narrow layer load a valid row
  };
  const int wcol0 = GU ? nb * kGateUpCols + 32 * wu : nb * kDownCols + 64 * wu;
  const bool active = wcol0 < N;

  // --- this wave's share of each stage's loads: wave-uniform bases + 32-bit offsets
  // A: MT*8 wave-loads of 1 KiB (4 rows each); wave takes v = wu + 8i, i < MT.  The
  // per-lane offsets stay below 2^31 bytes: a token row (gate/up) is at most 65535 x
  // 16384 x 2 bytes in; the h rows (down) are addressed from the M-block's first row,
  // which goes into the 64-bit base, so the offset is at most 159 x 4096 x 2 bytes.
  // W16: 2*MT wave-loads of 1 KiB (16 rows x 64 B each), v = wu + 8i for i < 2 while
  // v < 2 MT; row r's 16-byte chunk c at slot c ^ (r & 3).
  const char *abase = GU ? (const char *)a.x : (const char *)a.x + (size_t)row0 * I * 2;
  constexpr int NA = W16 ? 2 : MT;
  uint32_t aoff[NA];
  bool aon[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int v = wu + 8 * i;
    const int r = W16 ? 16 * v + (lane >> 2) : 4 * v + (lane >> 4);
    const int rl = min(r, rows - 1);
    const uint32_t row_elem = GU ? (uint32_t)a.row_token[row0 + rl] * (uint32_t)H : (uint32_t)rl * (uint32_t)I;
    const uint32_t chunk = W16 ? (uint32_t)((lane & 3) ^ (r & 3)) : (uint32_t)((lane & 15) ^ (r & 15));
    aoff[i] = 2u * (row_elem + 8u * chunk);
    aon[i] = !W16 || v < 2 * MT;
  }
  // B: 32 wave-loads of 1 KiB (16 slots x 64 B); wave takes v = wu + 8i, i < 4.  The 16
  // slots of a wave-load are 16 consecutive weight rows starting at a multiple of 16, so
  // in the tiled code layout each wave-load reads one contiguous KiB (the next step's is
  // the next KiB of the tile row).
  const char *bbase[4];
  uint32_t boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = wu + 8 * i;
    const int slot = 16 * v + (lane >> 2);
    bbase[i] = (const char *)slot_mat(16 * v).q;
    boff[i] = 4u * (uint32_t)code_index((size_t)slot_row(slot), 4 * ((lane & 3) ^ ((slot >> 2) & 3)), KF * K);
  }
  // S: 16 wave-loads of 256 B (64 slots x 2 groups): v < 8 scales, v >= 8 biases.
  // Wave-load v covers tile t = (v >> 2) & 1 of the wave pair m = v & 3, so its rows come
  // from one matrix.  Lane l takes the two rows 2(l%32), 2(l%32)+1 of those 64 (slot
  // 64 (2m + r/32) + 32 t + r%32 for r = 2(l%32)) in group 2ss + l/32: in the 16-row
  // tile layout the two values are adjacent, and the 16 lanes of one tile read the step's
  // 64-byte run.  In LDS, fp16 index 128 v + 64 (l/32) + r holds row r's group.  Wave wu
  // takes v = wu + 8i.
  const char *sbase[2];
  uint32_t soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = wu + 8 * i;
    const int t = (v >> 2) & 1, m = v & 3;
    const int r64 = 2 * (lane & 31);
    const int slot = 64 * (2 * m + (r64 >> 5)) + 32 * t + (r64 & 31);
    const QMat &M = slot_mat(32 * t);
    sbase[i] = (const char *)((v >> 3) ? M.b : M.s);
    const uint32_t n = (uint32_t)min(slot_row(slot), N - 2);
    soff[i] = 2u * (uint32_t)qp_index(n, lane >> 5, K / 64);
  }
  auto issue = [&](int ss, uint8_t *st) {
    const uint32_t l = lds_addr(st);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (aon[i]) dma16(abase + ss * (W16 ? 64 : 256), aoff[i], l + (wu + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(bbase[i] + ss * 1024, boff[i], l + kAStage + (wu + 8 * i) * 1024);
    if (!W16) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma4(sbase[i] + ss * (4 * kQpRows), soff[i], l + kAStage + kBStage + (wu + 8 * i) * 256);
    }
  };
  f32x16 acc[MT][2];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[t][i] = (f32x16){};

  // multiply one super-step (128 k) from stage `st`
  const int l15 = lane & 15;
  const int a_lane = (lane & 31) * kRowBytes;       // + t*32*256 (immediate) per row tile
  const int a_c0 = (hf * 8) ^ l15;                   // swizzled chunk of slice j: a_c0 ^ j
  int b_lane[2];                                     // this lane's weight slot per tile
  int s_lane[2];                                     // fp16 index of its scale (biases + 1024)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    b_lane[i] = (64 * wu + 32 * i + (lane & 31));
    s_lane[i] = 128 * ((i << 2) | (wu >> 1)) + 64 * hf + 32 * (wu & 1) + (lane & 31);
  }
  // bf16 weights: two 16-k slices per 32-k step, fragments straight from LDS
  auto compute16 = [&](const uint8_t *st) {
    const uint8_t *bb = st + kAStage;
    const int r = lane & 31;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 av[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        av[t] = *(const u32x4 *)(st + (t * 32 + r) * 64 + (((2 * j + hf) ^ (r & 3)) << 4));
      const u32x4 w0 = *(const u32x4 *)(bb + b_off(b_lane[0], 2 * j + hf));
      const u32x4 w1 = *(const u32x4 *)(bb + b_off(b_lane[1], 2 * j + hf));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w0),
                                                            __builtin_bit_cast(bf16x8, av[t]), acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w1),
                                                            __builtin_bit_cast(bf16x8, av[t]), acc[t][1], 0, 0, 0);
      }
    }
  };
  auto compute = [&](const uint8_t *st) {
    if (W16) {
      compute16(st);
      return;
    }
    const uint8_t *bb = st + kAStage;
    const uint16_t *sp = (const uint16_t *)(st + kAStage + kBStage);
    float sc[2], bi[2];
    DeqPair dp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sc[i] = qp_f32(sp[s_lane[i]], a.qbf16);
      bi[i] = qp_f32(sp[kSStage / 4 + s_lane[i]], a.qbf16);
      dp[i] = deq_pair(sc[i], bi[i]);
    }
    auto afrag = [&](int t, int j) {
      return *(const u32x4 *)(st + t * 32 * kRowBytes + a_lane + ((a_c0 ^ j) << 4));
    };
    // word j of the lane's 8 (16-byte part 2*hf + j/4, dword j%4) of its slot in tile i
    auto word = [&](int i, int j) {
      return *(const uint32_t *)(bb + b_off(b_lane[i], 2 * hf + (j >> 2)) + 4 * (j & 3));
    };
    // Software pipeline over the eight k-slices.  At the start of slice j the LDS reads
    // for later slices are issued as one group (activation fragments of slice j+1, packed
    // words of slice j+1 for tile 1 and j+2 for tile 0).  The slice's MFMAs run tile 0
    // first, then tile 1; tile 1's weights of slice j are dequantised between the tile-0
    // MFMAs and tile 0's weights of slice j+1 between the tile-1 MFMAs, so each tile needs
    // one register set of dequantised weights.
    u32x4 av[2][MT];
    uint32_t d0[4], d1[4];
#pragma unroll
    for (int t = 0; t < MT; ++t) av[0][t] = afrag(t, 0);
    dequant8_bf16_m(word(0, 0), dp[0], d0);
    uint32_t q1 = word(1, 0), q0 = word(0, 1);
    constexpr int kV = (20 + MT - 1) / MT;  // dequant VALU instructions per MFMA
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = j & 1, nx = c ^ 1;
      uint32_t n1 = 0, n0 = 0;
      if (j < 7) {
#pragma unroll
        for (int t = 0; t < MT; ++t) av[nx][t] = afrag(t, j + 1);
        n1 = word(1, j + 1);
      }
      if (j < 6) n0 = word(0, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      dequant8_bf16_m(q1, dp[1], d1);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t][0] = mfma(d0, av[c][t], acc[t][0]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (j < 7) dequant8_bf16_m(q0, dp[0], d0);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t][1] = mfma(d1, av[c][t], acc[t][1]);
      if (j < 7) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      q1 = n1;
      q0 = n0;
    }
  };
  // Two-stage ring, unrolled by two so each read names one stage object and the copies
  // in flight name the other.  The stage loads are issued from inline asm, so the
  // compiler adds no waits of its own for them; each wave waits for its loads, then the
  // barrier publishes every wave's.
  issue(ks0, stage0);
  if (!GU && 64 * wu < MT * 32) {
    // down: the rows' routing weights (read by the epilogue) go to LDS with the first
    // stage, so no register load and wait sits before the stage loads
    const int r = min(64 * wu + lane_now(), rows - 1);
    dma4(a.row_gate + row0, 4u * (uint32_t)r, lds_addr(s_gate) + 256 * wu);
  }
  // Down: the next item's ticket is taken by one thread as the item's last step begins,
  // so its round trip overlaps that step's multiplies; the value is read back by every
  // wave once the steps are done, when nothing else of the wave's is in flight (read
  // behind the epilogue's stores, its wait would also wait for them).  Gate/up (whose
  // registers do not hold the ticket through a step without spilling) takes it once the
  // last multiply is done and reads it back at the end of the epilogue.  The counter's
  // address carries a per-lane zero the compiler cannot see through, so it leaves the
  // atomic alone (with a uniform address it combines the lanes' adds and broadcasts the
  // result, waiting for the round trip at once).
  int pend = 0;
  auto take_ticket = [&]() {
    if (tid == 0 && claim) {
      uint32_t z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      pend = atomicAdd(claim + z, 1);
    }
  };
  for (int ss = ks0; ss < ks1; ss += 2) {
    vm_wait<0>();
    __syncthreads();  // stage0 holds step ss for every wave; stage1 is free
    if (ss + 1 < ks1) issue(ss + 1, stage1);
    if (!GU && ss + 1 == ks1) take_ticket();
    if (active) compute(stage0);
    if (ss + 1 >= ks1) break;
    vm_wait<0>();
    __syncthreads();  // stage1 holds step ss+1; stage0 is free
    if (ss + 2 < ks1) issue(ss + 2, stage0);
    if (!GU && ss + 2 == ks1) take_ticket();
    if (active) compute(stage1);
  }
  // every wave is past its last LDS read before the epilogue reuses stage0
  __builtin_amdgcn_s_barrier();
  if (GU)
    take_ticket();
  else
    pend = __builtin_amdgcn_readfirstlane(pend);  // the ticket (thread 0's), uniform
  if (GU && pc.ti >= 0) {
    // slot layout: per (wave, tile, matrix) 8 rows of 64 lanes of fp32 pairs, so each
    // store and load instruction covers 512 contiguous bytes
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const size_t wbase = (size_t)wu * MT * 2 * 512 + ln;
    if (active) {
      uint64_t *mine = a.part + ((size_t)pc.ti * pc.S + pc.p) * a.slot_u64 + wbase;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int h = 0; h < 8; ++h)
            st_agent(mine + (t * 2 + j) * 512 + h * 64,
                     ((uint64_t)__float_as_uint(acc[t][j][2 * h + 1]) << 32) | __float_as_uint(acc[t][j][2 * h]));
    }
    vm_drain();  // this thread's partial sums are stored (and the claim has returned)
    if (tid == 0) *s_pend = pend;
    __syncthreads();
    if (tid == 0) {
      const int c = ticket(a.tickets + pc.ti);
      *s_last = c == pc.S - 1;
      if (c == pc.S - 1) st_agent(a.tickets + pc.ti, 0);  // ready for the next launch
    }
    __syncthreads();
    if (!*s_last) return;
    if (active) {
      // one (tile, matrix) at a time: the S pieces' sums (this piece's own as stored) in
      // flight together, then added in piece order
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          asm volatile("" ::: "memory");  // keeps the groups' loads apart (register pressure)
          uint64_t v[kMaxSplit][8];
#pragma unroll
          for (int q = 0; q < kMaxSplit; ++q) {
            // pieces past S re-read the last slot; their terms are dropped below
            const uint64_t *src = a.part + ((size_t)pc.ti * pc.S + min(q, pc.S - 1)) * a.slot_u64 + wbase + (t * 2 + j) * 512;
#pragma unroll
            for (int h = 0; h < 8; ++h) v[q][h] = ld_agent(src + h * 64);
          }
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            float lo = __uint_as_float((uint32_t)v[0][h]), hi = __uint_as_float((uint32_t)(v[0][h] >> 32));
#pragma unroll
            for (int q = 1; q < kMaxSplit; ++q) {
              lo = q < pc.S ? lo + __uint_as_float((uint32_t)v[q][h]) : lo;
              hi = q < pc.S ? hi + __uint_as_float((uint32_t)(v[q][h] >> 32)) : hi;
            }
            acc[t][j][2 * h] = lo;
            acc[t][j][2 * h + 1] = hi;
          }
        }
    }
  }
  if (active) {
    // Epilogue, one 32-row tile at a time: the wave converts its tile to bf16 in its own
    // LDS area (GU: 32 rows x 32 h values; down: 32 rows x 64 gate-weighted outputs; rows
    // padded by 16 bytes so the 8-byte writes of 32 rows spread over the banks), then
    // writes whole row segments with 16-byte stores.
    constexpr int COLS = GU ? 32 : 64;
    constexpr int RB = COLS * 2 + 16;  // bytes per staged row
    uint8_t *tile = stage0 + wu * (32 * RB);
    // lane index made opaque here so its row/column arithmetic is not hoisted out of the
    // persistent loop (where it would occupy registers through the main loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 31, lh = ln >> 5;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float g = GU ? 1.0f : s_gate[t * 32 + lr];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GU) {
          float hv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float gv = acc[t][0][4 * q + u], uv = acc[t][1][4 * q + u];
            hv[u] = gv * sigmoid_fast(gv) * uv;
          }
          const uint2 pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *(uint2 *)(tile + lr * RB + 2 * (8 * q + 4 * lh)) = pk;
        } else {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const f32x16 &ac = acc[t][i];
            const uint2 pk = {pack_bf16x2(g * ac[4 * q], g * ac[4 * q + 1]),
                              pack_bf16x2(g * ac[4 * q + 2], g * ac[4 * q + 3])};
            *(uint2 *)(tile + lr * RB + 2 * (32 * i + 8 * q + 4 * lh)) = pk;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's tile writes are done
      constexpr int LPR = COLS / 8;        // lanes per row (16 B each)
      constexpr int RPI = 64 / LPR;        // rows per store instruction
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPI) {
        const int r = rr + ln / LPR;
        if (t * 32 + r < rows) {
          const uint4 v = *(const uint4 *)(tile + r * RB + 16 * (ln % LPR));
          uint16_t *dst = GU ? a.h + (size_t)(row0 + t * 32 + r) * I : a.y + (size_t)(row0 + t * 32 + r) * H;
          *(uint4 *)(dst + wcol0 + 8 * (ln % LPR)) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next tile overwrites
    }
  }
  if (tid == 0 && !(GU && pc.ti >= 0)) *s_pend = pend;
}

// Persistent grid.  Queue x serves M-blocks x, x+8, x+16, ... (all their N-blocks,
// consecutive); workgroup b starts on queue b % 8 (its XCD under round-robin
// dispatch) and moves on to the other queues when its own is empty.
//
// Gate/up: when the items fill their last round on the grid to at most half, that round
// would leave most workgroups idle while the rest run whole items.  Those last items (the
// M-blocks at the end of the block map, the shortest) are then split along K into S
// pieces (S <= 4, S * items <= workgroups) taken from one more queue after the others
// are empty, so the last round runs pieces of a fraction of an item each.
template <bool GU, bool W16>
__device__ __forceinline__ void run_item(const GemmArgs &a, uint8_t *stage0, uint8_t *stage1, float *s_gate,
                                         int *s_last, const int4 &mb, int nb, int ks0, int ks1, const Piece &pc,
                                         int *claim, int *s_pend, int wv0) {
  switch (mb.w) {
    case 1: gemm_item<1, GU, W16>(a, stage0, stage1, s_gate, s_last, mb.x, mb.y, mb.z, nb, ks0, ks1, pc, claim, s_pend, wv0); break;
    case 2: gemm_item<2, GU, W16>(a, stage0, stage1, s_gate, s_last, mb.x, mb.y, mb.z, nb, ks0, ks1, pc, claim, s_pend, wv0); break;
    case 3: gemm_item<3, GU, W16>(a, stage0, stage1, s_gate, s_last, mb.x, mb.y, mb.z, nb, ks0, ks1, pc, claim, s_pend, wv0); break;
    case 4: gemm_item<4, GU, W16>(a, stage0, stage1, s_gate, s_last, mb.x, mb.y, mb.z, nb, ks0, ks1, pc, claim, s_pend, wv0); break;
    default: gemm_item<5, GU, W16>(a, stage0, stage1, s_gate, s_last, mb.x, mb.y, mb.z, nb, ks0, ks1, pc, claim, s_pend, wv0); break;
  }
}

template <bool GU, bool W16>
__device__ void gemm_persistent(const GemmArgs &a) {
  // the wave's index (scalar) and, where needed, the lane's (mbcnt) are recomputed rather
  // than the thread index kept in a vector register for the whole kernel
  const int wv0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(16))) float s_gate[(kBM + 63) / 64 * 64];  // whole waves of 64
  __shared__ int s_item, s_queue, s_last, s_pend;
  // down: the first kMbCache block-map entries, copied once per launch, so an item finds
  // its entry without a round trip to memory (down runs about twice as many items per
  // workgroup as gate/up, which measured no better with the copy)
  constexpr int kMbCache = GU ? 1 : 384;
  __shared__ int4 s_mbc[kMbCache];
  const int NB = GU ? (a.I + kGateUpCols - 1) / kGateUpCols : (a.H + kDownCols - 1) / kDownCols;
  const int nss = (GU ? a.H : a.I) / (W16 ? 32 : 128);
  const int nmb = a.ctrl->n_mblocks;
  int m_cut = nmb, S = 1, n_tail = 0;
  if (GU && a.part) {
    const int P = gridDim.x, R = (NB * nmb) % P;
    if (R > 0 && 2 * R <= P) {
      const int mt = (R + NB - 1) / NB, ti = mt * NB;
      const int s = min(min(min(kMaxSplit, P / ti), nss), min(a.max_pieces / ti, kMaxTailItems / ti));
      if (s >= 2) {
        m_cut = nmb - mt;
        S = s;
        n_tail = ti;
      }
    }
  }
  auto items_of = [&](int x) { return m_cut > x ? NB * ((m_cut - x + kXcds - 1) / kXcds) : 0; };
  int cur = blockIdx.x % kXcds;  // wave 0: queue being drained (kXcds: the tail pieces)
  if (!GU)
    for (int i = (int)threadIdx.x; i < min(nmb, kMbCache); i += kGemmThreads) s_mbc[i] = a.mblocks[i];
  auto mblock = [&](int i) {  // after a barrier; wave-uniform, kept in scalar registers
    // The entry is uniform: an LDS read for the cached ones, else a scalar load.  Neither
    // is a vector memory load, so neither waits for the previous item's stores (a vector
    // or generic load here is followed by a wait that also covers every store in flight).
    u32x4 v;
    if (!GU && i < kMbCache) {
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(&s_mbc[i])) : "memory");
    } else {
      asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(a.mblocks + i) : "memory");
    }
    const int4 m = make_int4((int)v[0], (int)v[1], (int)v[2], (int)v[3]);
    return make_int4(__builtin_amdgcn_readfirstlane(m.x), __builtin_amdgcn_readfirstlane(m.y),
                     __builtin_amdgcn_readfirstlane(m.z), __builtin_amdgcn_readfirstlane(m.w));
  };
  int pq = -1;                    // wave 0: queue of the ticket in s_pend (-1: none)
  for (;;) {
    if (wv0 == 0) {
      // Claim the next unit.  The current queue first (one atomic); once it is empty, the
      // remaining counts of all eight queues are read in one round trip (one lane per
      // queue, atomic adds of zero, so the values are the queues' own) and the fullest
      // is taken; then the tail pieces.
      int lane = lane_now();
      asm volatile("" : "+v"(lane));  // per-lane values below are recomputed per claim, not kept
      int v = -1, q = -1;
      if (cur < kXcds) {
        int c = 0;
        if (lane == 0) c = pq == cur ? s_pend : atomicAdd(&a.queue[cur], 1);
        pq = -1;
        c = __builtin_amdgcn_readfirstlane(c);
        if (c < items_of(cur)) v = c, q = cur;
      }
      while (q < 0 && cur < kXcds) {
        int rem = 0, zero = 0;
        asm volatile("" : "+v"(zero));  // a real read-modify-write, not turned into a load
        if (lane < kXcds) rem = items_of(lane) - atomicAdd(&a.queue[lane], zero);
        int best = -1, best_rem = 0;
        for (int i = 0; i < kXcds; ++i) {
          const int r = __builtin_amdgcn_readlane(rem, i);
          if (r > best_rem) best_rem = r, best = i;
        }
        if (best < 0) {
          cur = kXcds;
          break;
        }
        cur = best;
        int c = 0;
        if (lane == 0) c = atomicAdd(&a.queue[cur], 1);
        c = __builtin_amdgcn_readfirstlane(c);
        if (c < items_of(cur)) v = c, q = cur;
      }
      if (q < 0 && n_tail) {
        int c = 0;
        if (lane == 0) c = pq == kXcds ? s_pend : atomicAdd(a.tail_queue, 1);
        pq = -1;
        c = __builtin_amdgcn_readfirstlane(c);
        if (c < n_tail * S) v = c, q = kXcds;
      }
      if (lane == 0) {
        s_item = v;
        s_queue = q;
      }
    }
    __syncthreads();
    const int v = __builtin_amdgcn_readfirstlane(s_item);  // uniform: keeps item state scalar
    const int q = __builtin_amdgcn_readfirstlane(s_queue);
    __syncthreads();
    if (v < 0) break;
    int4 mb;
    int nb, ks0 = 0, ks1 = nss;
    Piece pc{-1, 1, 0};
    if (q < kXcds) {
      mb = mblock(q + kXcds * (v / NB));
      nb = v % NB;
    } else {
      const int ti = v / S, p = v % S;
      mb = mblock(m_cut + ti / NB);
      nb = ti % NB;
      ks0 = p * nss / S;
      ks1 = (p + 1) * nss / S;
      pc = Piece{ti, S, p};
    }
    // the item takes the next ticket from the queue this one came from (the tail
    // pieces' queue for a piece)
    int *claim = q < kXcds ? &a.queue[q] : a.tail_queue;
    run_item<GU, W16>(a, stage0, stage1, s_gate, &s_last, mb, nb, ks0, ks1, pc, claim, &s_pend, wv0);
    cur = q;
    pq = q;
  }
}

__global__ __launch_bounds__(kGemmThreads) void k_gemm_gateup(GemmArgs a) { gemm_persistent<true, false>(a); }
__global__ __launch_bounds__(kGemmThreads) void k_gemm_down(GemmArgs a) { gemm_persistent<false, false>(a); }
__global__ __launch_bounds__(kGemmThreads) void k_gemm_gateup_w16(GemmArgs a) { gemm_persistent<true, true>(a); }
__global__ __launch_bounds__(kGemmThreads) void k_gemm_down_w16(GemmArgs a) { gemm_persistent<false, true>(a); }

// MOE_F_SEPARATE_DEQUANT: a stack of `rows` packed matrix rows (K columns, the tiled
// code and scale/bias layouts) expanded to bf16 (w = s*q + b in fp32, rounded to nearest
// even) in tiles of 16 rows x 32 k (1 KB; 16-byte chunk c4 of row r of tile (n16, tk) at
// ((n16*(K/32) + tk)*16 + r)*4 + c4).  One thread per 16-byte output chunk (one code word).
__global__ __launch_bounds__(256) void k_dequant_w16(const uint32_t *__restrict__ q, const uint16_t *__restrict__ sc,
                                                     const uint16_t *__restrict__ bi, uint4 *__restrict__ dst,
                                                     int64_t total, int K, bool qbf16) {
  const int tpr = K / 32;  // tiles per row
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t tile = i >> 6;
    const int within = (int)(i & 63), r = within >> 2, c4 = within & 3;
    const int64_t n16 = tile / tpr;
    const int tk = (int)(tile - n16 * tpr);
    const size_t n = (size_t)(n16 * 16 + r);
    const uint32_t w = q[code_index(n, 4 * tk + c4, K)];
    const size_t qi = qp_index(n, (32 * tk + 8 * c4) / 64, K / 64);
    const float s = qp_f32(sc[qi], qbf16), b = qp_f32(bi[qi], qbf16);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(__builtin_fmaf(s, (float)((w >> (8 * j)) & 0xfu), b),
                         __builtin_fmaf(s, (float)((w >> (8 * j + 4)) & 0xfu), b));
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Combine: out[t] = sum over the NR = k+1 grouped rows of token t (already
// gate-weighted), fp32 sum in slot order, bf16 result.  One workgroup per token, eight
// columns per thread; the token's row indices go through LDS and all NR row loads of a
// thread are issued before the first is summed.
template <int NR>
__global__ __launch_bounds__(256) void k_finalize(const uint16_t *y, const int32_t *slot_row, uint16_t *out, int H) {
  __shared__ int s_rows[NR];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < NR) s_rows[threadIdx.x] = slot_row[(size_t)t * NR + threadIdx.x];
  __syncthreads();
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    uint4 v[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) v[j] = *(const uint4 *)(y + (size_t)s_rows[j] * H + 8 * c);
    float acc[8] = {};
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_lo(w[i]);
        acc[2 * i + 1] += bf16_hi(w[i]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *(uint4 *)(out + (size_t)t * H + 8 * c) = o;
  }
}

template <int NR>
hipError_t launch_fin(const uint16_t *y, const int32_t *slot_row, uint16_t *out, int T, int H, int nr, hipStream_t s) {
  if constexpr (NR > kMaxTopK + 1) {
    return hipErrorInvalidValue;
  } else {
    if (nr != NR) return launch_fin<NR + 1>(y, slot_row, out, T, H, nr, s);
    hipLaunchKernelGGL(k_finalize<NR>, dim3(T), dim3(256), 0, s, y, slot_row, out, H);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_gemm_gateup(const GemmArgs &a, int n_blocks, hipStream_t s) {
  if (a.w16)
    hipLaunchKernelGGL(k_gemm_gateup_w16, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm_gateup, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs &a, int n_blocks, hipStream_t s) {
  if (a.w16)
    hipLaunchKernelGGL(k_gemm_down_w16, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm_down, dim3(n_blocks), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequant_w16(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, void *dst, int64_t rows,
                              int K, bool qbf16, hipStream_t s) {
  const int64_t total = rows * (int64_t)(K / 8);
  const int64_t want = (total + 255) / 256;
  hipLaunchKernelGGL(k_dequant_w16, dim3((int)(want < 16384 ? want : 16384)), dim3(256), 0, s, q, sc, bi, (uint4 *)dst,
                     total, K, qbf16);
  return hipGetLastError();
}

hipError_t launch_finalize(const uint16_t *y, const int32_t *slot_row, uint16_t *out, int T, int H, int k,
                           hipStream_t s) {
  return launch_fin<2>(y, slot_row, out, T, H, k + 1, s);
}

}  // namespace moe
