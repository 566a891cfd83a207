/*
 * moe.h -- C ABI of the MI355X sparse mixture-of-experts feed-forward layer.
 *
 * The layer ("Optimizing on-device inference for Apple Silicon", section "Qwen
 * creates three different workload shapes"): a router scores E routed experts
 * per token and keeps the top k; one shared expert processes every token.  Each
 * expert is a SwiGLU feed-forward block whose weights are stored as 4-bit codes
 * with one scale and one bias per group of 64 weights (section "Prefill >
 * Dequantize weights during matmul").  The layer output is
 *
 *     out[t] = sum_{e in S_t} g_{t,e} * FFN_e(x_t) + c_t * FFN_shared(x_t)
 *     FFN(v) = W_down * (silu(W_gate v) .* (W_up v)),   silu(a) = a*sigmoid(a)
 *
 * with S_t the k experts of largest router logit l[t][e] = x_t . Wr[e] (+ b[e])
 * -- equal logits: the lower expert index wins -- and g_{t,.} the softmax of
 * the chosen logits; c_t = 1, or sigmoid(x_t . w_sg) with the optional shared-expert gate
 * vector w_sg.  Logits are ranked as if computed exactly; the library
 * certifies its fp32 ranking against a rigorous error bound and re-ranks
 * uncertain tokens in binary64 (sequentially summed, ascending h, when even
 * that cannot separate them).
 *
 * Two forms (section "Optimization strategy", first part: a matrix path for
 * prefill, a vector path for batch-1 decode):
 *   moe_forward_prefill -- T tokens: router, on-device histogram / prefix scan
 *     / scatter / block map (section "Prefill > Keep expert routing on the
 *     GPU"), grouped GEMMs that dequantise int4 tiles on chip and feed bf16
 *     MFMA with fp32 accumulation, tile height chosen from each expert's row
 *     count (section "Prefill > Match tile size to expert load"), SwiGLU fused
 *     into the gate/up GEMM, gate-weighted combine fused into the down GEMM,
 *     long prompts processed in bounded chunks (section "Prefill > Bound
 *     temporary memory with prompt chunking");
 *   moe_forward_decode -- one token: row-parallel dequant-GEMV over the k+1
 *     active experts (section "Decode > Optimize the one-row weight path") with
 *     the two input projections and the activation fused, and the output
 *     projection fused with the routing weights and the shared expert (section
 *     "Decode > Reduce intermediate and state traffic").
 *
 * Conventions
 *   - Every pointer argument is a DEVICE pointer unless marked (host).
 *   - The caller owns all device memory: weights, x, out and the workspace.  A
 *     plan holds a host copy of the config and of the weight pointers only; it
 *     allocates no device memory and launches nothing.  Weights must stay valid
 *     and unmodified for the plan's lifetime.
 *   - Forwards only enqueue work on `stream` (0 = null stream) and never
 *     synchronise the host.  Device-side faults surface at the caller's next
 *     synchronisation.  Calls that may run concurrently need distinct
 *     workspaces.  A plan is immutable and may be shared between threads.
 *   - Errors: host validation returns a status before anything is enqueued; a
 *     failed launch returns MOE_ERR_HIP (hipGetLastError() is left for the
 *     caller).  No C++ exception crosses this interface.
 *   - x and out must not alias.  x, out, router weight and code arrays must be
 *     16-byte aligned, scale/bias arrays 8-byte aligned, the workspace 256-byte aligned.
 *
 * Layouts (row-major unless stated):
 *   x, out           bf16 [T][H]
 *   router weight    [E][H], bf16 (MOE_BF16) or float32 (MOE_FP32)
 *   router bias      float32 [E], or NULL
 *   quantised W[N][K]  q: uint32 words in tiles of 16 rows x 128 k: element k of
 *                    row n is the 4-bit code in bits 4*(k%8) (low nibble first) of
 *                    word ((n/16)*(K/128) + k/128)*256 + (n%16)*16 + (k%128)/8, so a
 *                    128-k step of 16 rows is one run of 1 KB (moe_pack_codes
 *                    converts row-major [N][K/8] words);
 *                    w = scale*code + bias with one fp16 (or bf16) scale and bias per row
 *                    n and group g = k/64, stored in 16-row tiles: the pair of
 *                    (n, g) is element ((n/16)*(K/64) + g)*16 + n%16 of the
 *                    scale and of the bias array (moe_pack_qparams converts
 *                    row-major [N][K/64] arrays).  A tile holds 64 B per group
 *                    pair, so a 128-k step of 16 rows reads one run of 64 B.
 *   routed experts   stacked: gate, up [E][I][H]; down [E][H][I] (q, scale
 *                    and bias each stacked on the leading axis)
 *   shared expert    gate, up [I][H]; down [H][I]
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* unsupported sizes (see moe_config) */
  MOE_ERR_DTYPE = 3,     /* unsupported dtype */
  MOE_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  MOE_ERR_TOKENS = 6,    /* T < 1 (prefill) */
  MOE_ERR_DEVICE = 7,    /* current device is not gfx950, or device query failed */
  MOE_ERR_HIP = 8,       /* a kernel launch failed */
  MOE_ERR_ALIAS = 9,     /* x and out (or a pack's src and dst) overlap */
  MOE_ERR_ALLOC = 10,    /* host allocation failed */
  MOE_ERR_WAIT = 11      /* moe_workspace_check: an internal decode wait ran out of polls
                            since the workspace was initialised; outputs of the decode
                            calls since then are not valid */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_FP16 = 1, MOE_FP32 = 2 } moe_dtype;

/* Flags (moe_config.flags).  Section "Optimization strategy" of the pages measures each
 * optimisation against an otherwise identical configuration without it; the flags
 * below select such configurations.  Unknown bits are rejected (MOE_ERR_SHAPE).
 *
 * MOE_F_FORCE_BM(rows): every M-block of the grouped GEMMs is `rows` tall (32, 64, 96,
 *   128 or 160; the last block of an expert holds the remainder) instead of a height
 *   picked from the expert's row count (section "Prefill > Match tile size to expert
 *   load": the ablation fixes the tile size).  The smallest tile the grouped GEMM has is
 *   one 32 x 32 MFMA tile, so MOE_F_FORCE_BM(32) is the fixed-small-tile configuration.
 * MOE_F_NO_FALLBACK: prefill keeps the fp32 top-k of a token even when its error bound
 *   does not certify it (no binary64 re-rank).  Routing may then differ from the exact
 *   ranking; for tests and timing only.  No effect with a float32 router (ranked in
 *   binary64 throughout) or on decode.
 * MOE_F_SEPARATE_DEQUANT: each prefill call first expands the weights of all E+1
 *   experts into bf16 matrices in the workspace, and the grouped GEMMs read those instead
 *   of the packed codes (section "Prefill > Dequantize weights during matmul": the
 *   ablation expands the 4-bit weights into a bf16 array that the matrix kernel reads
 *   back).  The workspace grows by (E+1) * 3 * I * H * 2 bytes (1.6 GB at H = 2048,
 *   I = 512, E = 256).
 * MOE_F_HOST_ROUTING: prefill stops after grouping each chunk, synchronises the stream
 *   on the host, reads the block-map length and launches the grouped GEMMs with exactly
 *   one workgroup per work item (section "Prefill > Keep expert routing on the GPU": the
 *   ablation lets the CPU inspect the routing before the next launch).  The forward then
 *   blocks the host; the stream must not be under graph capture. */
#define MOE_F_NONE 0u
#define MOE_F_FORCE_BM(rows) ((uint32_t)((rows) / 32) & 0xfu)
#define MOE_F_NO_FALLBACK (1u << 4)
#define MOE_F_SEPARATE_DEQUANT (1u << 5)
#define MOE_F_HOST_ROUTING (1u << 6)

typedef struct {               /* (host) */
  int32_t hidden;              /* H: multiple of 256, <= 16384 */
  int32_t inter;               /* I: intermediate size of every expert (routed and
                                  shared); multiple of 128, <= 4096 */
  int32_t n_experts;           /* E: 1 <= E <= 256 */
  int32_t top_k;               /* k: 1 <= k <= min(E, 16) */
  int32_t group_size;          /* must be 64 */
  moe_dtype router_dtype;      /* MOE_BF16 or MOE_FP32 */
  moe_dtype qparam_dtype;      /* scale/bias dtype: MOE_FP16, or MOE_BF16 (the pages'
                                  checkpoint format) */
  int32_t max_chunk_tokens;    /* prefill chunk; fixes the workspace size; 1..65536 */
  uint32_t flags;              /* MOE_F_* bits; unknown bits -> MOE_ERR_SHAPE */
} moe_config;

typedef struct {               /* (host struct of device pointers) */
  const uint32_t *q;           /* N*K/8 code words in 16 x 128 tiles */
  const void *scale;           /* fp16, N*K/64 values in 16-row tiles */
  const void *bias;            /* fp16, same layout */
} moe_qmat;

typedef struct {               /* (host struct of device pointers) */
  const void *router_w;        /* [E][H] bf16 or float32 */
  const float *router_bias;    /* [E] or NULL */
  moe_qmat gate, up;           /* routed, [E][I][H] */
  moe_qmat down;               /* routed, [E][H][I] */
  moe_qmat s_gate, s_up;       /* shared, [I][H] */
  moe_qmat s_down;             /* shared, [H][I] */
  const void *shared_gate;     /* bf16 [H], 16-byte aligned, or NULL.  If given, the shared
                                  expert's output is weighted by sigmoid(x_t . shared_gate)
                                  (fp32 sum of the exact products); NULL: weight 1 */
} moe_weights;

typedef struct moe_plan_s *moe_plan_t;

/* Prefill stages (indices into moe_debug_out.events). */
enum {
  MOE_STAGE_ROUTE = 0,   /* logits, top-k, gates, certification, fp64 re-rank */
  MOE_STAGE_GROUP = 1,   /* histogram, prefix scan, scatter, block map */
  MOE_STAGE_GATEUP = 2,  /* grouped GEMM gate/up + SwiGLU */
  MOE_STAGE_DOWN = 3,    /* grouped GEMM down + gate-weighted combine */
  MOE_STAGE_FINAL = 4,   /* per token: sum of its k+1 gate-weighted rows -> bf16 */
  MOE_PREFILL_STAGES = 5
};
/* Decode stages: the whole token (logits, top-k, gates, gate/up GEMV + SwiGLU,
 * down GEMV + routing weights + shared expert) is one launch. */
enum {
  MOE_DSTAGE_LAYER = 0,
  MOE_DECODE_STAGES = 1
};

/* Optional diagnostics of one forward (any field may be NULL).
 * For prefill with T > max_chunk_tokens, topk_ids/gates cover all T tokens;
 * counts/offsets are per chunk, concatenated ([n_chunks][E+1], [n_chunks][E+2]);
 * row_token is per chunk, chunk c's rows starting at c*max_chunk_tokens*(k+1)
 * and holding chunk-local token indices; n_refined[c] counts chunk c's tokens
 * whose fp32 ranking was not certified and were re-ranked in binary64.
 * events (host array of hipEvent_t): if non-NULL it must hold n_stages+1
 * events; event i is recorded on the stream before stage i and event n_stages
 * after the last stage (of the last chunk). */
typedef struct {
  int32_t *topk_ids;           /* [T][k], ascending expert index per token */
  float *gates;                /* [T][k], gate of topk_ids[t][j] */
  int32_t *counts;             /* [n_chunks][E+1]; bin E = shared expert */
  int32_t *offsets;            /* [n_chunks][E+2] */
  int32_t *row_token;          /* [n_chunks * max_chunk_tokens * (k+1)] */
  int32_t *n_refined;          /* [n_chunks] */
  hipEvent_t *events;          /* (host) */
  float *logits32;             /* [T][E] prefill, bf16 router only: the fp32 logits (+ bias)
                                  that the selection ranks first (left untouched otherwise) */
  float *radii32;              /* [T][E] prefill, bf16 router only: the certified bound on
                                  |logits32 - exact logit| used by that ranking */
} moe_debug_out;

/* Validate cfg and w (host checks only: no device work, no device memory) and
 * create a plan.  *workspace_bytes receives the workspace size every forward
 * with this plan needs (it depends only on cfg).  Queries the current device
 * once; it must be a gfx950. */
moe_status moe_plan_create(const moe_config *cfg, const moe_weights *w, moe_plan_t *plan,
                           size_t *workspace_bytes);
void moe_plan_destroy(moe_plan_t plan);

/* Initialise a workspace's control words (enqueued on stream).  Required once
 * per workspace before its first forward; forwards leave it initialised. */
moe_status moe_workspace_init(moe_plan_t plan, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Read the workspace's decode error word (enqueued on stream, then the host waits for
 * stream): MOE_OK if every decode call on this workspace since moe_workspace_init
 * completed its internal hand-offs, MOE_ERR_WAIT if a wait ran out of polls (the word
 * stays set until moe_workspace_init), MOE_ERR_HIP if the copy failed.  Blocks the host.
 * workspace NULL: the array of moe_forward_decode_static on the current device (the
 * word stays set for the life of the process). */
moe_status moe_workspace_check(moe_plan_t plan, const void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Prefill: x, out bf16 [T][H]; T >= 1.  Tokens are processed in chunks of at
 * most max_chunk_tokens with one workspace. */
moe_status moe_forward_prefill(moe_plan_t plan, const void *x, int64_t T, void *out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream,
                               const moe_debug_out *dbg);

/* Decode: one token; x, out bf16 [H].  One launch whose workgroups hand results to
 * each other inside the launch (section "Decode > Keep every decode step on the
 * GPU"); requires E <= 256.  If an internal wait ever exceeded its poll budget, the
 * control word at byte offset 88 of the workspace (int32) becomes non-zero (the output of
 * that call is then invalid); moe_workspace_init clears it.  The hand-off records are
 * tagged with a per-call number drawn from call counters in the workspace (every call
 * advances them by the same amount, whatever its grid), so the launch arguments depend
 * only on (plan, x, out, workspace, dbg): a sequence of decode calls may
 * be captured once in a HIP graph and replayed, also interleaved with direct calls on the
 * same workspace, as long as the calls on one workspace stay ordered on one stream.
 * Workgroups of the launch wait for each other, so the launch must have the GPU to
 * itself: a concurrent kernel that occupies compute units can delay the waits until they
 * run out of polls (check with moe_workspace_check). */
moe_status moe_forward_decode(moe_plan_t plan, const void *x, void *out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream,
                              const moe_debug_out *dbg);

/* Decode of a small batch: T rows (1 <= T <= 8, e.g. the draft tokens a speculative
 * decoder verifies at once; section "Limits of further optimization": batches of 2-5
 * rows are an inefficient shape for one-row kernels and read experts again).  x, out
 * bf16 [T][H].  Same layer, routing and numerics per row as moe_forward_decode (which
 * is this call with T = 1), in one launch that reads each active expert's weights once
 * -- the union of the rows' experts -- and applies them to every row that chose the
 * expert.  debug topk_ids / gates are [T][k].  MOE_ERR_TOKENS if T is out of range;
 * other errors and the graph-capture property as moe_forward_decode. */
moe_status moe_forward_decode_batch(moe_plan_t plan, const void *x, int32_t T, void *out, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream, const moe_debug_out *dbg);

/* Decode without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and result as moe_forward_decode, with the control block and
 * the decode's records, intermediate values and counters in a device array inside the
 * library (2 MiB per device, held until the process ends) instead of a workspace.
 * Allocates nothing: no hipMalloc, no hipFree, no allocating library call.  The first
 * call on a device enqueues a kernel on `stream` that clears the array.
 * MOE_ERR_WORKSPACE if the plan's one-token decode records (192E + 16(k+1)I bytes, plus
 * alignment and 2 KB of counters) do not fit the array (never for sizes
 * moe_plan_create accepts today: at most 0.65 MB).  Every call on a GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams, different threads) race and
 * must be ordered by the caller.  moe_workspace_check(plan, NULL, 0, stream) reads this
 * array's error word.  Other errors as moe_forward_decode. */
moe_status moe_forward_decode_static(moe_plan_t plan, const void *x, void *out, hipStream_t stream,
                                     const moe_debug_out *dbg);

/* Weight preparation: rewrite an fp16 array of one value per (row, group of 64)
 * from row-major src [rows][k/64] into the 16-row tile layout the quantised
 * matrices use (element (n, g) to ((n/16)*(k/64) + g)*16 + n%16) in dst (enqueued
 * on stream).  rows: a multiple of 16 (a stack of experts' matrices may be packed
 * in one call: every N here is a multiple of 16, so tiles never straddle two
 * experts); k: a positive multiple of 64.  src and dst are device arrays of
 * rows*k/64 fp16, 4-byte aligned, and must not overlap.  MOE_ERR_NULL,
 * MOE_ERR_SHAPE (rows < 16 or not a multiple of 16, k not a positive multiple of
 * 64), MOE_ERR_ALIGN, MOE_ERR_ALIAS (overlap) or MOE_ERR_HIP. */
moe_status moe_pack_qparams(const void *src, void *dst, int64_t rows, int32_t k,
                            hipStream_t stream);

/* Weight preparation: rewrite row-major 4-bit code words src [rows][k/8] (element k
 * of row n in bits 4*(k%8) of word k/8) into the tile layout of the quantised
 * matrices (word w of row n to ((n/16)*(k/128) + w/16)*256 + (n%16)*16 + w%16) in dst
 * (enqueued on stream).  rows: a multiple of 16 (a stack of experts' matrices may be
 * packed in one call); k: a positive multiple of 128.  src and dst are device arrays
 * of rows*k/8 uint32, 16-byte aligned, and must not overlap.  MOE_ERR_NULL,
 * MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_ALIAS or MOE_ERR_HIP. */
moe_status moe_pack_codes(const uint32_t *src, uint32_t *dst, int64_t rows, int32_t k,
                          hipStream_t stream);

const char *moe_status_string(moe_status s);

/* Library build identification, e.g. "moe-mi355x gfx950". */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
