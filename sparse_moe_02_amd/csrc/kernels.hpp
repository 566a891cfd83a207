// Launch interfaces of the MoE kernels (host side calls these from api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kRouteTokens = 32;   // tokens per router workgroup
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kBM = 160;           // max rows of one grouped-GEMM M-block (5 MFMA row tiles)
constexpr int kGemmThreads = 512;  // grouped GEMM workgroup: 8 waves, two per SIMD
constexpr int kGateUpCols = 256;   // h columns per gate/up work item (8 waves x 32)
constexpr int kDownCols = 512;     // output columns per down work item (8 waves x 64)

struct QMat {
  const uint32_t *q;
  const uint16_t *s;
  const uint16_t *b;
};

constexpr int kMaxTailItems = 1024;  // split gate/up tail items per launch (<= workgroups / 2)
constexpr int kMaxSplit = 4;         // pieces per split gate/up item
constexpr int kPartSlots = 256;      // partial-sum slots provided at least (when y is smaller)
constexpr size_t kStaticScratchBytes = size_t(2) << 20;  // moe_forward_decode_static's device array
constexpr int kXcds = 8;           // MI355X: 8 accelerator complex dies, one L2 each

// Control words at the start of the workspace.
struct Ctrl {
  int pad0;
  int n_mblocks;         // M-blocks in the block map
  int n_refined;         // tokens re-ranked in binary64 this chunk (reset by the group kernel)
  int pad1;
  int q_gateup[kXcds];   // grouped GEMM work queues, one per XCD (reset by the group kernel)
  int q_down[kXcds];
  int q_tail;            // gate/up tail-piece queue (reset by the group kernel)
  int pad2;
  int d_err;             // decode: a wait ran out of polls (sticky; cleared by workspace init)
  int pad3[2];
  int pad[39];
};
static_assert(sizeof(Ctrl) == 256, "control block is one 256-byte slot");
static_assert(__builtin_offsetof(Ctrl, d_err) == 88, "documented offset of the decode error word");

struct RouteArgs {
  const uint16_t *x;      // [T][H] bf16 (chunk)
  const uint16_t *wr16;   // [E][H] bf16 router (or null)
  const float *wr32;      // [E][H] fp32 router (or null)
  const float *bias;      // [E] or null
  int T, H, E, k;
  int32_t *ids;           // [T][k] ascending
  float *gates;           // [T][k]
  uint32_t *tokmask;      // [ceil(T/32)][256] bit m: token 32*blk+m chose e (0 for e >= E)
  float *lg, *rd;         // [T][E] fp32 logits (+bias) and their error radii (bf16 router)
  Ctrl *ctrl;
  int32_t *dbg_ids;       // optional [T][k] (chunk-offset)
  float *dbg_gates;
  bool no_fallback;       // keep uncertified fp32 selections (MOE_F_NO_FALLBACK)
};

struct GroupArgs {
  const int32_t *ids;
  const float *gates;
  const uint32_t *tokmask;
  int T, E, k;
  int32_t *counts;        // [E+1]
  int32_t *offsets;       // [E+2]
  int32_t *row_token;     // [T*(k+1)]
  float *row_gate;        // [T*(k+1)]
  int32_t *slot_row;      // [T][k+1] grouped row of (token, slot); slot k = shared
  int4 *mblocks;          // {expert, row0, rows, mt}
  Ctrl *ctrl;
  int32_t *dbg_counts, *dbg_offsets, *dbg_row_token, *dbg_n_refined;
  int force_rows;         // 0: M-block heights from the expert's row count; else fixed height
  const float *sgate;     // [T] shared-expert weight per token, or null (weight 1)
};

struct GemmArgs {
  const uint16_t *x;        // gate/up: activations [T][H]; down: h [rows][I]
  const int4 *mblocks;
  const Ctrl *ctrl;
  int *queue;               // kXcds counters
  int *tail_queue;          // gate/up: counter of claimed tail pieces
  uint64_t *part;           // gate/up: fp32 partial sums of split tail items (null: no split)
  int *tickets;             // gate/up: pieces finished per split tail item (zero between launches)
  int max_pieces;           // partial-sum slots that fit in `part`
  int slot_u64;             // 8-byte words per slot: 32 rows x 2 x kGateUpCols fp32 per MT
  const int32_t *row_token;
  const float *row_gate;
  QMat w0, w1;              // routed stacked (gate, up) or (down, -)
  QMat s0, s1;              // shared expert
  int E, H, I;
  bool qbf16;               // scale/bias are bf16 (else fp16)
  bool w16;                 // w0/w1/s0/s1 .q are bf16 matrices (16 x 32 tiles), no scale/bias
  uint16_t *h;              // gate/up output [rows][I]
  uint16_t *y;              // down output, gate-weighted, per grouped row [rows][H]
};

constexpr int kMaxDecodeT = 8;     // tokens of one decode call (a verification batch)
constexpr int kDecGuTask = 16;     // rows of one decode gate/up task
constexpr int kDecDnTask = 64;     // output rows of one decode down task
constexpr int kCtrStride = 64;     // ints between two completion counters (256 bytes)
constexpr int kLrecRep = 8;        // copies of the one-token kernel's logit records
constexpr int kHrecRep = 4;        // copies of the one-token kernel's h records

struct DecodeArgs {
  const uint16_t *x;        // [T][H]
  const uint16_t *wr16;
  const float *wr32;
  const float *bias;
  QMat gate, up, down;      // routed stacked
  QMat s_gate, s_up, s_down;
  int H, E, k, I, T;
  bool qbf16;               // scale/bias are bf16 (else fp16)
  const uint16_t *sgate;    // [H] bf16 shared-expert gate vector, or null (weight 1)
  uint64_t *lrec;           // [T][E][3] tagged records: low and high word of the binary64 logit, radius
                            // (one-token kernel: [kLrecRep][E][3], copies of the same records)
  uint64_t *srec;           // [T][2k] tagged records: the chosen experts (ascending), then their gates
  uint64_t *hflag;          // [min(T*k, E) + 1][I/16] tagged: gate/up task (active expert, row block) done
  float *hval;              // [T][k+1][I] h of every (token, slot); slot k = shared expert
  uint64_t *hrec1;          // one-token kernel: [kHrecRep][(k+1)*I/2] tagged pairs of bf16 h values
  float *part;              // [T][k+1][H] gate-weighted down output of every (token, slot)
  int *rbctr;               // [T][H/64] arrivals per (token, row block), kCtrStride ints apart
  uint64_t *epctr;          // [8] call counters (epoch_ticket), kCtrStride ints apart
  Ctrl *ctrl;
  uint16_t *out;            // [T][H]
  int32_t *dbg_ids;         // [T][k]
  float *dbg_gates;
};

// Decode workspace regions, in bytes, for T <= t_max tokens (offsets from a 256-byte
// aligned base; each region 256-byte aligned).  t_max = 1: only the regions of the
// one-token kernel (lrec, hrec1, epctr; the other offsets are 0 and unused).
struct DecodeLayout {
  size_t lrec, srec, hflag, hval, hrec1, part, rbctr, epctr, total;
};
DecodeLayout decode_layout(int H, int E, int k, int I, int t_max);

hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_group(const GroupArgs &a, hipStream_t s);
// out[t] = sigmoid(x[t] . w) for the T tokens of x [T][H] (bf16), w [H] (bf16)
hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *w, float *out, int T, int H, hipStream_t s);
hipError_t launch_gemm_gateup(const GemmArgs &a, int n_blocks, hipStream_t s);
hipError_t launch_gemm_down(const GemmArgs &a, int n_blocks, hipStream_t s);
// Expand a stack of packed matrices (rows x K) into bf16 16 x 32 tiles at dst.
hipError_t launch_dequant_w16(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, void *dst, int64_t rows,
                              int K, bool qbf16, hipStream_t s);
hipError_t launch_finalize(const uint16_t *y, const int32_t *slot_row, uint16_t *out, int T, int H, int k,
                           hipStream_t s);
// Workgroups that may be resident at once for the decode kernel of up to t_max tokens
// (all of its workgroups wait for each other, so its grid never exceeds this).
int decode_capacity(int t_max, int n_cu);
int decode_grid(const DecodeArgs &a, int capacity);  // workgroups of one decode launch
hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t s);
// The one-token kernel (decode1.hip): logits, selection and h as tagged records.
int decode1_capacity(int n_cu);
int decode1_grid(const DecodeArgs &a, int capacity);
hipError_t launch_decode1(const DecodeArgs &a, int grid, hipStream_t s);
hipError_t launch_ctrl_init(Ctrl *c, void *clear, size_t clear_bytes, hipStream_t s);

// Gated DeltaNet prefill scan (gdn.hip): heads of width kGdnDim.
constexpr int kGdnDim = 128;
struct GdnArgs {
  const uint16_t *q, *k;    // [T][hk][128] bf16
  const uint16_t *v;        // [T][hv][128] bf16
  const float *alpha, *beta;  // [T][hv]
  float *state;             // [hv][128][128] fp32, in: S_0, out: S_T
  uint16_t *out;            // [T][hv][128] bf16
  int T, hk, hv;
};
hipError_t launch_gdn_scan(const GdnArgs &a, hipStream_t s);
hipError_t launch_pack_qparams(const uint16_t *src, uint16_t *dst, int64_t rows, int G, hipStream_t s);
hipError_t launch_pack_codes(const uint32_t *src, uint32_t *dst, int64_t rows, int K, hipStream_t s);

}  // namespace moe
