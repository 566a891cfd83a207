// Host side of the C ABI declared in include/moe.h: validation, workspace layout, the
// prefill chunk loop ("Optimizing on-device inference for Apple Silicon", section
// "Prefill > Bound temporary memory with prompt chunking") and the launch sequences.
// Every step is enqueued on the caller's stream with no host synchronisation in
// between (section "Prefill > Keep expert routing on the GPU").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>

#include "../../include/moe.h"
#include "../../include/gdn.h"
#include "kernels.hpp"

using namespace moe;

struct moe_plan_s {
  moe_config cfg;
  moe_weights w;
  int n_cu;
  int dec_cap[4];  // batch-decode workgroups that fit at once, for up to 2, 2, 4, 8 tokens
  int dec1_cap;    // the same for the one-token kernel
  DecodeLayout dec;         // decode regions inside the workspace (up to 8 tokens), from off_dec
  DecodeLayout dec_static;  // the same for one token, inside the static scratch (after 256 B)
  // workspace layout (byte offsets)
  size_t slot_u64;  // 8-byte words per partial-sum slot of a split gate/up piece
  size_t off_ctrl, off_tokmask, off_lg, off_rd, off_ids, off_gates, off_counts, off_offsets, off_row_token,
      off_row_gate, off_slot_row, off_mblocks, off_sgate, off_h, off_y, off_dec, off_tk, off_dend, off_w16, total;
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// M-block height forced by MOE_F_FORCE_BM (0: chosen from each expert's row count)
int forced_rows(uint32_t flags) { return 32 * (int)(flags & 0xfu); }

constexpr uint32_t kKnownFlags = 0xfu | MOE_F_NO_FALLBACK | MOE_F_SEPARATE_DEQUANT | MOE_F_HOST_ROUTING;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_qmat(const moe_qmat &m) {
  if (!m.q || !m.scale || !m.bias) return MOE_ERR_NULL;
  if (!aligned16(m.q)) return MOE_ERR_ALIGN;
  if (((uintptr_t)m.scale & 7u) || ((uintptr_t)m.bias & 7u)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

void layout(moe_plan_s &p) {
  const size_t C = (size_t)p.cfg.max_chunk_tokens, E = p.cfg.n_experts, k = p.cfg.top_k;
  const size_t H = p.cfg.hidden, I = p.cfg.inter;
  const size_t nblk = (C + kRouteTokens - 1) / kRouteTokens;
  const size_t rows = C * (k + 1);
  const size_t bm = forced_rows(p.cfg.flags) ? (size_t)forced_rows(p.cfg.flags) : (size_t)kBM;
  const size_t max_mblocks = rows / bm + E + 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  p.off_ctrl = take(sizeof(Ctrl));
  p.off_tokmask = take(nblk * kMaxExperts * 4);
  p.off_lg = take(C * E * 4);
  p.off_rd = take(C * E * 4);
  p.off_ids = take(C * k * 4);
  p.off_gates = take(C * k * 4);
  p.off_counts = take((E + 1) * 4);
  p.off_offsets = take((E + 2) * 4);
  p.off_row_token = take(rows * 4);
  p.off_row_gate = take(rows * 4);
  p.off_slot_row = take(rows * 4);
  p.off_mblocks = take(max_mblocks * 16);
  p.off_sgate = take(C * 4);  // shared-expert weight per token (with a gate vector)
  p.off_h = take(rows * I * 2);
  // y also holds the partial sums of split gate/up items (before the down GEMM writes y):
  // at least kPartSlots slots, one per piece, sized for the tallest M-block of a chunk
  const size_t mt_max = (std::min<size_t>(kBM, C) + 31) / 32;
  p.slot_u64 = mt_max * 32 * 2 * kGateUpCols / 2;
  const size_t nb_gu = (I + kGateUpCols - 1) / kGateUpCols;
  const size_t part = std::min<size_t>(kMaxSplit * nb_gu * max_mblocks, kPartSlots) * p.slot_u64 * 8;
  p.off_y = take(std::max(rows * H * 2, part));
  // decode records and counters (cleared by moe_workspace_init), then the split-item
  // tickets of the gate/up GEMM (zero between launches)
  p.dec = decode_layout((int)H, (int)E, (int)k, (int)I, kMaxDecodeT);
  p.dec_static = decode_layout((int)H, (int)E, (int)k, (int)I, 1);
  p.off_dec = take(p.dec.total);
  p.off_tk = take(kMaxTailItems * 4);
  p.off_dend = o;
  // MOE_F_SEPARATE_DEQUANT: every expert's gate, up and down matrices expanded to bf16
  p.off_w16 = o;
  if (p.cfg.flags & MOE_F_SEPARATE_DEQUANT) take((E + 1) * 3 * I * H * 2);
  p.total = o;
}

template <class T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

QMat qm(const moe_qmat &m) {
  return QMat{m.q, static_cast<const uint16_t *>(m.scale), static_cast<const uint16_t *>(m.bias)};
}

moe_status check_ws(const moe_plan_s *p, void *ws, size_t bytes) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (bytes < p->total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return MOE_ERR_ALIGN;
  return MOE_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// gfx950 check of the current device, cached per device (plan-free entry points)
constexpr int kMaxDevs = 64;
std::atomic<int> g_dev_ok[kMaxDevs];  // 0 unknown, 1 gfx950, 2 other
moe_status current_device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevs) return MOE_ERR_DEVICE;
  int ok = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(ok, std::memory_order_relaxed);
  }
  return ok == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

hipError_t rec(const moe_debug_out *dbg, int i, hipStream_t s) {
  if (dbg && dbg->events) return hipEventRecord(dbg->events[i], s);
  return hipSuccess;
}

// One decode launch of T tokens over the given control block and decode regions (L:
// offsets from `base`).
moe_status decode_launch(const moe_plan_s *p, const void *x, int T, void *out, Ctrl *ctrl, char *base,
                         const DecodeLayout &L, hipStream_t stream, const moe_debug_out *dbg) {
  const moe_config &c = p->cfg;
  DecodeArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  const bool fp32_router = c.router_dtype == MOE_FP32;
  a.wr16 = fp32_router ? nullptr : static_cast<const uint16_t *>(p->w.router_w);
  a.wr32 = fp32_router ? static_cast<const float *>(p->w.router_w) : nullptr;
  a.bias = p->w.router_bias;
  a.gate = qm(p->w.gate);
  a.up = qm(p->w.up);
  a.down = qm(p->w.down);
  a.s_gate = qm(p->w.s_gate);
  a.s_up = qm(p->w.s_up);
  a.s_down = qm(p->w.s_down);
  a.H = c.hidden;
  a.E = c.n_experts;
  a.k = c.top_k;
  a.I = c.inter;
  a.T = T;
  a.qbf16 = c.qparam_dtype == MOE_BF16;
  a.sgate = static_cast<const uint16_t *>(p->w.shared_gate);
  a.lrec = reinterpret_cast<uint64_t *>(base + L.lrec);
  a.srec = reinterpret_cast<uint64_t *>(base + L.srec);
  a.hflag = reinterpret_cast<uint64_t *>(base + L.hflag);
  a.hval = reinterpret_cast<float *>(base + L.hval);
  a.hrec1 = reinterpret_cast<uint64_t *>(base + L.hrec1);
  a.part = reinterpret_cast<float *>(base + L.part);
  a.rbctr = reinterpret_cast<int *>(base + L.rbctr);
  a.epctr = reinterpret_cast<uint64_t *>(base + L.epctr);
  a.ctrl = ctrl;
  a.out = static_cast<uint16_t *>(out);
  if (dbg) {
    a.dbg_ids = dbg->topk_ids;
    a.dbg_gates = dbg->gates;
  }
  const int cap = p->dec_cap[T <= 1 ? 0 : T <= 2 ? 1 : T <= 4 ? 2 : 3];
  if (rec(dbg, MOE_DSTAGE_LAYER, stream) != hipSuccess) return MOE_ERR_HIP;
  const hipError_t e = T == 1 ? launch_decode1(a, decode1_grid(a, p->dec1_cap), stream)
                              : launch_decode(a, decode_grid(a, cap), stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (rec(dbg, MOE_DECODE_STAGES, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

// ------------------------------------------------------------ static decode scratch
// moe_forward_decode_static keeps the decode's control block and its records, h values,
// partial outputs and counters in this file-scope device array instead of a caller
// workspace: [0, 256) the control block, then the one-token decode regions.  Each device
// holds its own copy; host code uses only the address hipGetSymbolAddress returns for the
// current device (the array's name is a host-side stand-in).  The first call on a device
// clears the array with a kernel on the caller's stream; later calls rely on the decode
// protocol itself (a fresh tag per call from counters that only grow).
constexpr size_t kStaticDec = 256;

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
char *g_static_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// Address of this device's scratch (set up on the first call on the device).
moe_status static_scratch(hipStream_t stream, char **base) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    char *b = static_cast<char *>(ptr);
    if (launch_ctrl_init(reinterpret_cast<Ctrl *>(b), b + kStaticDec, kStaticScratchBytes - kStaticDec, stream) !=
        hipSuccess)
      return MOE_ERR_HIP;
    g_static_ptr[dev] = b;
  }
  *base = g_static_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "unsupported shape or flags";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_ALIGN: return "pointer not aligned (16 B; scale/bias 8 B; workspace 256 B)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_TOKENS: return "token count out of range";
    case MOE_ERR_DEVICE: return "current device is not gfx950 or cannot be queried";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_ALIAS: return "input and output arrays overlap";
    case MOE_ERR_ALLOC: return "host allocation failed";
    case MOE_ERR_WAIT: return "a decode wait ran out of polls; decode outputs since the workspace init are invalid";
  }
  return "unknown status";
}

const char *moe_version(void) { return "moe-mi355x gfx950 1"; }

moe_status moe_pack_codes(const uint32_t *src, uint32_t *dst, int64_t rows, int32_t k, hipStream_t stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (rows < 16 || rows % 16 != 0 || k < 128 || k % 128 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  const uintptr_t bytes = (uintptr_t)rows * (uintptr_t)(k / 8) * 4u;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_ALIAS;
  if (moe::launch_pack_codes(src, dst, rows, k, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_pack_qparams(const void *src, void *dst, int64_t rows, int32_t k, hipStream_t stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (rows < 16 || rows % 16 != 0 || k < 64 || k % 64 != 0) return MOE_ERR_SHAPE;
  if (((uintptr_t)src & 3u) || ((uintptr_t)dst & 3u)) return MOE_ERR_ALIGN;
  const uintptr_t bytes = (uintptr_t)rows * (uintptr_t)(k / 64) * 2u;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_ALIAS;
  if (moe::launch_pack_qparams(static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), rows, k / 64,
                               stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_plan_create(const moe_config *cfg, const moe_weights *w, moe_plan_t *plan,
                           size_t *workspace_bytes) {
  if (!cfg || !w || !plan) return MOE_ERR_NULL;
  *plan = nullptr;
  const moe_config &c = *cfg;
  if (c.group_size != 64) return MOE_ERR_SHAPE;
  if (c.hidden < 256 || c.hidden > 16384 || c.hidden % 256) return MOE_ERR_SHAPE;
  if (c.inter < 128 || c.inter > 4096 || c.inter % 128) return MOE_ERR_SHAPE;
  if (c.n_experts < 1 || c.n_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > kMaxTopK) return MOE_ERR_SHAPE;
  if (c.max_chunk_tokens < 1 || c.max_chunk_tokens > 65536) return MOE_ERR_SHAPE;
  if ((c.flags & ~kKnownFlags) != 0 || forced_rows(c.flags) > kBM) return MOE_ERR_SHAPE;
  if (c.router_dtype != MOE_BF16 && c.router_dtype != MOE_FP32) return MOE_ERR_DTYPE;
  if (c.qparam_dtype != MOE_FP16 && c.qparam_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (!w->router_w) return MOE_ERR_NULL;
  if (!aligned16(w->router_w) || (w->router_bias && ((uintptr_t)w->router_bias & 3u))) return MOE_ERR_ALIGN;
  if (w->shared_gate && !aligned16(w->shared_gate)) return MOE_ERR_ALIGN;
  for (const moe_qmat *m : {&w->gate, &w->up, &w->down, &w->s_gate, &w->s_up, &w->s_down}) {
    const moe_status st = check_qmat(*m);
    if (st != MOE_OK) return st;
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return MOE_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
  moe_plan_s *p = new (std::nothrow) moe_plan_s();
  if (!p) return MOE_ERR_ALLOC;
  p->cfg = c;
  p->w = *w;
  p->n_cu = prop.multiProcessorCount;
  for (int v = 0; v < 4; ++v) p->dec_cap[v] = decode_capacity(1 << v, p->n_cu);
  p->dec1_cap = decode1_capacity(p->n_cu);
  layout(*p);
  if (workspace_bytes) *workspace_bytes = p->total;
  *plan = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t plan) { delete plan; }

moe_status moe_workspace_init(moe_plan_t p, void *ws, size_t bytes, hipStream_t stream) {
  if (!p) return MOE_ERR_NULL;
  const moe_status st = check_ws(p, ws, bytes);
  if (st != MOE_OK) return st;
  return launch_ctrl_init(at<Ctrl>(ws, p->off_ctrl), at<char>(ws, p->off_dec), p->off_dend - p->off_dec, stream) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status moe_workspace_check(moe_plan_t p, const void *ws, size_t bytes, hipStream_t stream) {
  if (!p) return MOE_ERR_NULL;
  const char *ctrl = nullptr;
  if (ws) {
    const moe_status st = check_ws(p, const_cast<void *>(ws), bytes);
    if (st != MOE_OK) return st;
    ctrl = static_cast<const char *>(ws) + p->off_ctrl;
  } else {  // the static scratch of moe_forward_decode_static on the current device
    char *b = nullptr;
    const moe_status st = static_scratch(stream, &b);
    if (st != MOE_OK) return st;
    ctrl = b;
  }
  int32_t word = 0;
  if (hipMemcpyAsync(&word, ctrl + offsetof(Ctrl, d_err), sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_ERR_HIP;
  return word ? MOE_ERR_WAIT : MOE_OK;
}

moe_status moe_forward_prefill(moe_plan_t p, const void *x, int64_t T, void *out, void *ws, size_t bytes,
                               hipStream_t stream, const moe_debug_out *dbg) {
  if (!p || !x || !out) return MOE_ERR_NULL;
  if (T < 1 || T > ((int64_t)1 << 40)) return MOE_ERR_TOKENS;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
  moe_status st = check_ws(p, ws, bytes);
  if (st != MOE_OK) return st;
  const moe_config &c = p->cfg;
  const size_t H = c.hidden, E = c.n_experts, k = c.top_k;
  if (overlap(x, (size_t)T * H * 2, out, (size_t)T * H * 2)) return MOE_ERR_ALIAS;
  const int64_t C = c.max_chunk_tokens;
  const int gemm_blocks = p->n_cu;  // persistent: one 8-wave workgroup per CU
  Ctrl *ctrl = at<Ctrl>(ws, p->off_ctrl);
  const bool fp32_router = c.router_dtype == MOE_FP32;

  // MOE_F_SEPARATE_DEQUANT: expand the weights to bf16 first (the grouped GEMMs then read
  // those): routed stacks to experts 0..E-1, the shared expert to expert E
  const bool w16 = (c.flags & MOE_F_SEPARATE_DEQUANT) != 0;
  const size_t I = c.inter, mat16 = I * H;  // bf16 elements of one matrix
  uint16_t *g16 = at<uint16_t>(ws, p->off_w16), *u16 = g16 + (E + 1) * mat16, *d16 = u16 + (E + 1) * mat16;
  if (w16) {
    const bool qb = c.qparam_dtype == MOE_BF16;
    struct {
      const moe_qmat &m;
      uint16_t *dst;
      int64_t rows;
      int K;
    } jobs[6] = {{p->w.gate, g16, (int64_t)E * c.inter, c.hidden},
                 {p->w.up, u16, (int64_t)E * c.inter, c.hidden},
                 {p->w.down, d16, (int64_t)E * c.hidden, c.inter},
                 {p->w.s_gate, g16 + E * mat16, c.inter, c.hidden},
                 {p->w.s_up, u16 + E * mat16, c.inter, c.hidden},
                 {p->w.s_down, d16 + E * mat16, c.hidden, c.inter}};
    for (const auto &j : jobs)
      if (launch_dequant_w16(j.m.q, static_cast<const uint16_t *>(j.m.scale), static_cast<const uint16_t *>(j.m.bias),
                             j.dst, j.rows, j.K, qb, stream) != hipSuccess)
        return MOE_ERR_HIP;
  }
  auto bf16_mat = [&](uint16_t *base) { return QMat{reinterpret_cast<const uint32_t *>(base), nullptr, nullptr}; };

  for (int64_t c0 = 0, ci = 0; c0 < T; c0 += C, ++ci) {
    const int Tc = (int)((T - c0 < C) ? (T - c0) : C);
    const bool last = c0 + C >= T;
    const moe_debug_out *d = last ? dbg : nullptr;
    const uint16_t *xc = static_cast<const uint16_t *>(x) + (size_t)c0 * H;
    uint16_t *oc = static_cast<uint16_t *>(out) + (size_t)c0 * H;

    RouteArgs ra{};
    ra.x = xc;
    ra.wr16 = fp32_router ? nullptr : static_cast<const uint16_t *>(p->w.router_w);
    ra.wr32 = fp32_router ? static_cast<const float *>(p->w.router_w) : nullptr;
    ra.bias = p->w.router_bias;
    ra.T = Tc;
    ra.H = (int)H;
    ra.E = (int)E;
    ra.k = (int)k;
    ra.ids = at<int32_t>(ws, p->off_ids);
    ra.gates = at<float>(ws, p->off_gates);
    ra.tokmask = at<uint32_t>(ws, p->off_tokmask);
    ra.lg = at<float>(ws, p->off_lg);
    ra.rd = at<float>(ws, p->off_rd);
    ra.ctrl = ctrl;
    ra.no_fallback = (c.flags & MOE_F_NO_FALLBACK) != 0;
    if (dbg) {
      ra.dbg_ids = dbg->topk_ids ? dbg->topk_ids + (size_t)c0 * k : nullptr;
      ra.dbg_gates = dbg->gates ? dbg->gates + (size_t)c0 * k : nullptr;
    }
    if (rec(d, MOE_STAGE_ROUTE, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_route(ra, stream) != hipSuccess) return MOE_ERR_HIP;
    if (dbg && !fp32_router) {
      const size_t n = (size_t)Tc * E * sizeof(float);
      if (dbg->logits32 &&
          hipMemcpyAsync(dbg->logits32 + (size_t)c0 * E, ra.lg, n, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return MOE_ERR_HIP;
      if (dbg->radii32 &&
          hipMemcpyAsync(dbg->radii32 + (size_t)c0 * E, ra.rd, n, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return MOE_ERR_HIP;
    }

    GroupArgs ga{};
    ga.ids = ra.ids;
    ga.gates = ra.gates;
    ga.tokmask = ra.tokmask;
    ga.T = Tc;
    ga.E = (int)E;
    ga.k = (int)k;
    ga.counts = at<int32_t>(ws, p->off_counts);
    ga.offsets = at<int32_t>(ws, p->off_offsets);
    ga.row_token = at<int32_t>(ws, p->off_row_token);
    ga.row_gate = at<float>(ws, p->off_row_gate);
    ga.slot_row = at<int32_t>(ws, p->off_slot_row);
    ga.mblocks = at<int4>(ws, p->off_mblocks);
    ga.ctrl = ctrl;
    ga.force_rows = forced_rows(c.flags);
    if (p->w.shared_gate) {
      ga.sgate = at<float>(ws, p->off_sgate);
      if (launch_shared_gate(xc, static_cast<const uint16_t *>(p->w.shared_gate), at<float>(ws, p->off_sgate), Tc,
                             (int)H, stream) != hipSuccess)
        return MOE_ERR_HIP;
    }
    if (dbg) {
      ga.dbg_counts = dbg->counts ? dbg->counts + (size_t)ci * (E + 1) : nullptr;
      ga.dbg_offsets = dbg->offsets ? dbg->offsets + (size_t)ci * (E + 2) : nullptr;
      ga.dbg_row_token = dbg->row_token ? dbg->row_token + (size_t)c0 * (k + 1) : nullptr;
      ga.dbg_n_refined = dbg->n_refined ? dbg->n_refined + ci : nullptr;
    }
    if (rec(d, MOE_STAGE_GROUP, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_group(ga, stream) != hipSuccess) return MOE_ERR_HIP;

    // persistent grid of one workgroup per CU; with MOE_F_HOST_ROUTING the host waits for
    // the block map and launches one workgroup per work item instead
    int grid_gu = gemm_blocks, grid_dn = gemm_blocks;
    if (c.flags & MOE_F_HOST_ROUTING) {
      int nmb = 0;
      if (hipMemcpyAsync(&nmb, &ctrl->n_mblocks, sizeof(nmb), hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess)
        return MOE_ERR_HIP;
      const int nb_gu = (c.inter + kGateUpCols - 1) / kGateUpCols, nb_dn = (c.hidden + kDownCols - 1) / kDownCols;
      grid_gu = std::max(1, nmb * nb_gu);
      grid_dn = std::max(1, nmb * nb_dn);
    }

    GemmArgs g1{};
    g1.x = xc;
    g1.mblocks = ga.mblocks;
    g1.ctrl = ctrl;
    g1.queue = ctrl->q_gateup;
    g1.row_token = ga.row_token;
    g1.row_gate = ga.row_gate;
    g1.w0 = qm(p->w.gate);
    g1.w1 = qm(p->w.up);
    g1.s0 = qm(p->w.s_gate);
    g1.s1 = qm(p->w.s_up);
    g1.E = (int)E;
    g1.H = (int)H;
    g1.I = c.inter;
    g1.qbf16 = c.qparam_dtype == MOE_BF16;
    g1.w16 = w16;
    if (w16) {
      g1.w0 = bf16_mat(g16);
      g1.w1 = bf16_mat(u16);
      g1.s0 = bf16_mat(g16 + E * mat16);
      g1.s1 = bf16_mat(u16 + E * mat16);
    }
    g1.h = at<uint16_t>(ws, p->off_h);
    // the partial sums of split gate/up items live in y, which only the down GEMM writes
    g1.tail_queue = &ctrl->q_tail;
    g1.part = at<uint64_t>(ws, p->off_y);
    g1.max_pieces = (int)std::min<size_t>((p->off_dec - p->off_y) / (p->slot_u64 * 8), 1 << 20);
    g1.slot_u64 = (int)p->slot_u64;
    g1.tickets = at<int>(ws, p->off_tk);
    if (rec(d, MOE_STAGE_GATEUP, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm_gateup(g1, grid_gu, stream) != hipSuccess) return MOE_ERR_HIP;

    GemmArgs g2 = g1;
    g2.x = g1.h;
    g2.queue = ctrl->q_down;
    g2.w0 = w16 ? bf16_mat(d16) : qm(p->w.down);
    g2.s0 = w16 ? bf16_mat(d16 + E * mat16) : qm(p->w.s_down);
    g2.w1 = QMat{};
    g2.s1 = QMat{};
    g2.y = at<uint16_t>(ws, p->off_y);
    g2.part = nullptr;
    if (rec(d, MOE_STAGE_DOWN, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm_down(g2, grid_dn, stream) != hipSuccess) return MOE_ERR_HIP;

    if (rec(d, MOE_STAGE_FINAL, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_finalize(g2.y, ga.slot_row, oc, Tc, (int)H, (int)k, stream) != hipSuccess) return MOE_ERR_HIP;
    if (rec(d, MOE_PREFILL_STAGES, stream) != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_forward_decode(moe_plan_t p, const void *x, void *out, void *ws, size_t bytes, hipStream_t stream,
                              const moe_debug_out *dbg) {
  return moe_forward_decode_batch(p, x, 1, out, ws, bytes, stream, dbg);
}

moe_status moe_forward_decode_batch(moe_plan_t p, const void *x, int32_t T, void *out, void *ws, size_t bytes,
                                    hipStream_t stream, const moe_debug_out *dbg) {
  if (!p || !x || !out) return MOE_ERR_NULL;
  if (T < 1 || T > kMaxDecodeT) return MOE_ERR_TOKENS;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
  moe_status st = check_ws(p, ws, bytes);
  if (st != MOE_OK) return st;
  const moe_config &c = p->cfg;
  const size_t n = (size_t)T * c.hidden * 2;
  if (overlap(x, n, out, n)) return MOE_ERR_ALIAS;
  return decode_launch(p, x, T, out, at<Ctrl>(ws, p->off_ctrl), at<char>(ws, p->off_dec), p->dec, stream, dbg);
}

moe_status moe_forward_decode_static(moe_plan_t p, const void *x, void *out, hipStream_t stream,
                                     const moe_debug_out *dbg) {
  if (!p || !x || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
  const moe_config &c = p->cfg;
  if (overlap(x, (size_t)c.hidden * 2, out, (size_t)c.hidden * 2)) return MOE_ERR_ALIAS;
  if (kStaticDec + p->dec_static.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  char *base = nullptr;
  const moe_status st = static_scratch(stream, &base);
  if (st != MOE_OK) return st;
  return decode_launch(p, x, 1, out, reinterpret_cast<Ctrl *>(base), base + kStaticDec, p->dec_static, stream, dbg);
}

moe_status moe_gdn_scan(int32_t T, int32_t n_kheads, int32_t n_vheads, int32_t d_k, int32_t d_v, const void *q,
                        const void *k, const void *v, const float *alpha, const float *beta, float *state,
                        void *out, hipStream_t stream) {
  if (T < 0) return MOE_ERR_TOKENS;
  if (d_k != kGdnDim || d_v != kGdnDim) return MOE_ERR_SHAPE;
  if (n_kheads < 1 || n_vheads < 1 || n_vheads > 4096 || n_vheads % n_kheads != 0) return MOE_ERR_SHAPE;
  if (!state) return MOE_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return MOE_ERR_NULL;
  if (!aligned16(state)) return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || ((uintptr_t)alpha & 3u) ||
                ((uintptr_t)beta & 3u) || ((uintptr_t)out & 1u)))
    return MOE_ERR_ALIGN;
  const size_t nqk = (size_t)T * n_kheads * kGdnDim * 2, nv = (size_t)T * n_vheads * kGdnDim * 2;
  const size_t ng = (size_t)T * n_vheads * 4, ns = (size_t)n_vheads * kGdnDim * kGdnDim * 4;
  if (T > 0) {
    // the output and the state may overlap no input and not each other
    for (const auto &w : {std::make_pair((const void *)out, nv), std::make_pair((const void *)state, ns)})
      if (overlap(w.first, w.second, q, nqk) || overlap(w.first, w.second, k, nqk) ||
          overlap(w.first, w.second, v, nv) || overlap(w.first, w.second, alpha, ng) ||
          overlap(w.first, w.second, beta, ng))
        return MOE_ERR_ALIAS;
    if (overlap(out, nv, state, ns)) return MOE_ERR_ALIAS;
  }
  const moe_status st = current_device_ok();
  if (st != MOE_OK) return st;
  GdnArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.alpha = alpha;
  a.beta = beta;
  a.state = state;
  a.out = static_cast<uint16_t *>(out);
  a.T = T;
  a.hk = n_kheads;
  a.hv = n_vheads;
  return launch_gdn_scan(a, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
