"""Benchmark of the MoE layer on one MI355X.

One step = one 4096-token prefill of the uniform-routing layer (hidden 2048, 256 experts
top-8 + 1 shared, intermediate 512, int4 group-64 weights) followed by a batch-1 decode
sweep over 40 distinct weight sets of the same shape (so decode weights stream from HBM,
not from cache).  Inputs are resident in HBM before timing starts.

Prints one JSON line: value = prefill tokens/s; also decode microseconds per layer, the
per-stage times from HIP events recorded by the library on its stream, roofline figures
for the dominant kernel of each form (against the datasheet peaks and against ceilings
measured in the same run), the skewed-routing prefill, the 128K chunked prompt, and the
oracle's CPU throughput on the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 4K prefill + decode µs/layer; % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill4k_decode40_hbm_traffic.md")


def profiled_traffic(kernel):
    """HBM bytes per dispatch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE profile
    (scaled by the copy-kernel calibration it records), or None when the kernel sources have
    changed since the counters were taken."""
    import hashlib

    try:
        lines = open(TRAFFIC_PROFILE).read().split("\n")
    except OSError:
        return None
    srcs, want, val = [], None, None
    for line in lines:
        f = line.split()
        if len(f) >= 2 and f[0] == "sources:":
            srcs = f[1:]
        elif len(f) == 2 and f[0] == "sources_sha256:":
            want = f[1]
        elif len(f) == 3 and f[0] == "traffic_bytes" and f[1] == kernel:
            val = float(f[2])
    if not srcs or want is None or val is None:
        return None
    h = hashlib.sha256()
    for s in srcs:
        with open(os.path.join(ROOT, s), "rb") as fh:
            h.update(fh.read())
    return val if h.hexdigest() == want else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def mblock_rows(counts, force_rows=0, bm=160):
    """The grouped GEMMs' M-blocks for one chunk's expert counts (the block-map rule of the
    grouping kernel): balanced blocks of at most `bm` rows, or blocks of `force_rows` and one
    remainder block.  Returns (rows of every block, MFMA tile rows of every block)."""
    rows = []
    for n in (int(c) for c in counts):
        if n == 0:
            continue
        if force_rows:
            nmb = -(-n // force_rows)
            rows += [force_rows] * (nmb - 1) + [n - (nmb - 1) * force_rows]
        else:
            nmb = -(-n // bm)
            q, rem = divmod(n, nmb)
            rows += [q + 1] * rem + [q] * (nmb - rem)
    rows = np.array(rows)
    return rows, 32 * ((rows + 31) // 32)


def time_events(fn, reps, stream, B):
    """Run fn() reps times with HIP events between runs on `stream`; per-run ms."""
    import torch

    ev = B.HipEvents(reps + 1)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for i in range(reps):
        fn()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    return np.array([ev.elapsed_ms(i, i + 1) for i in range(reps)])


def ceilings(dev, stream, B, dec_layers, dec_x, H, I, k):
    """Measured reference points: HBM read stream, MFMA loop, launch cost, and the decode
    step's nine-expert weight stream with the experts already known (with and without the
    dequant arithmetic)."""
    import torch

    from sparse_moe_02_amd import probes

    out = {}
    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    for grid in (2048, 4096):
        probes.read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream)
    ms = time_events(lambda: probes.read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), 4096, stream), 5, stream, B)
    out["hbm_read_GBs"] = round(nbytes / (float(np.min(ms)) * 1e-3) / 1e9, 1)
    del buf
    iters, grid = 4000, 1024  # 4 waves per workgroup: 4 waves per SIMD
    flop = grid * 4 * iters * 4 * (2 * 32 * 32 * 16)
    probes.mfma(100, sink.data_ptr(), grid, stream)
    ms = time_events(lambda: probes.mfma(iters, sink.data_ptr(), grid, stream), 3, stream, B)
    out["mfma_bf16_TFLOPs"] = round(flop / (float(np.min(ms)) * 1e-3) / 1e12, 1)
    # the same instruction on random bf16 operands (real data switches more bits and the
    # chip draws more power: the clock the GEMMs actually run at), and the grouped GEMM's
    # register pipeline (two words dequantised per 2 x 5 MFMAs) without its LDS traffic
    gen = torch.Generator(device="cpu").manual_seed(0)
    ngrid = 512
    src = (torch.randn(ngrid * 8 * 64 * 8, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
    iters = 2000
    probes.mfma_data(src.data_ptr(), 20, sink.data_ptr(), ngrid, stream)
    ms = time_events(lambda: probes.mfma_data(src.data_ptr(), iters, sink.data_ptr(), ngrid, stream), 3, stream, B)
    out["mfma_bf16_random_data_TFLOPs"] = round(ngrid * 8 * iters * 10 * 32768 / (float(np.min(ms)) * 1e-3) / 1e12, 1)
    iters = 250
    probes.dequant_mfma(src.data_ptr(), 5, sink.data_ptr(), ngrid, stream)
    ms = time_events(lambda: probes.dequant_mfma(src.data_ptr(), iters, sink.data_ptr(), ngrid, stream), 3, stream, B)
    out["dequant_mfma_pipeline_TFLOPs"] = round(ngrid * 8 * iters * 80 * 32768 / (float(np.min(ms)) * 1e-3) / 1e12, 1)
    del src

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        return g

    n = 40
    g1 = graph_of(lambda: probes.empty(1, 64, torch.cuda.current_stream().cuda_stream), n)
    ms = time_events(g1.replay, 10, stream, B)
    out["empty_kernel_graph_us"] = round(float(np.median(ms)) * 1e3 / n, 3)
    g2 = graph_of(lambda: probes.empty(288, 256, torch.cuda.current_stream().cuda_stream), n)
    ms = time_events(g2.replay, 10, stream, B)
    out["empty_kernel_288x256_graph_us"] = round(float(np.median(ms)) * 1e3 / n, 3)
    del g1, g2
    if dec_layers:
        # the experts each decode layer's token chose, from one debug call per layer
        mats, tables = [], []
        for m, x in zip(dec_layers, dec_x):
            _, d = m.decode(x, debug=True)
            ids = d["topk_ids"].cpu().numpy()[0].tolist() + [m.E]
            p, nb = [], []
            for e in ids:
                for name in ("gate", "up", "down"):
                    for part in ("_q", "_s", "_b"):
                        t = m.t[name + part][e]
                        p.append(t.data_ptr())
                        nb.append(t.numel() * t.element_size())
            mats.append(p)
            rw = m.t["router_w"]
            tab, fgrid = probes.flat_table(p + [rw.data_ptr()], nb + [rw.numel() * rw.element_size()])
            tables.append((torch.from_numpy(tab.view(np.int64)).to(dev), len(p) + 1, fgrid))

        # the same bytes (nine experts + router) as one flat read, routing given: the floor
        # of a single-phase decode layer
        def flat_sweep():
            s = torch.cuda.current_stream().cuda_stream
            for tab, n, fgrid in tables:
                probes.flat_stream(tab.data_ptr(), n, sink.data_ptr(), fgrid, s)
        g = graph_of(flat_sweep, 1)
        ms = time_events(g.replay, 10, stream, B)
        out["layer_bytes_flat_stream_us"] = round(float(np.median(ms)) * 1e3 / len(tables), 3)
        del g
        for arith in (True, False):
            def sweep(arith=arith):
                s = torch.cuda.current_stream().cuda_stream
                for p, x in zip(mats, dec_x):
                    probes.expert_stream(p, x.data_ptr(), H, I, arith, sink.data_ptr(), 1024, s)
            g = graph_of(sweep, 1)
            ms = time_events(g.replay, 10, stream, B)
            # the decode GEMVs' access pattern with the experts known: with the arithmetic,
            # and with it replaced by an XOR of the loaded words
            key = "expert_gemv_stream_us" if arith else "expert_gemv_stream_no_arith_us"
            out[key] = round(float(np.median(ms)) * 1e3 / len(mats), 3)
            del g
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-layers", type=int, default=40)
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed decode sweep")
    ap.add_argument("--no-long-prompt", action="store_true", help="skip the 131072-token chunked prefill")
    ap.add_argument("--no-skewed", action="store_true", help="skip the skewed-routing prefill")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured ceilings")
    ap.add_argument("--no-ablations", action="store_true", help="skip the ablation configurations")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet prefill scan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(calibrates the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from sparse_moe_02_amd import binding as B
    from sparse_moe_02_amd.layer import MoeLayer, bf16_tensor

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return
    sh2 = synth.shape_of(2)
    T, H, I, E, k = sh2.T, sh2.H, sh2.I, sh2.E, sh2.k

    log("bench: drawing the prefill layer")
    Lp = synth.make_layer(2)
    xp_bits = synth.make_x(2)
    pre = MoeLayer(Lp, top_k=k, max_chunk_tokens=T, device=dev)
    xp = bf16_tensor(xp_bits, dev)
    outp = torch.empty_like(xp)

    n_dec = 0 if args.prefill_only else args.decode_layers
    dec_layers, dec_x, dec_out = [], [], []
    Lb = None
    for li in range(n_dec):
        Lb = synth.make_layer(1, li, into=Lb)
        dec_layers.append(MoeLayer(Lb, top_k=k, max_chunk_tokens=1, device=dev))
        dec_x.append(bf16_tensor(synth.make_x(1, li)[0], dev))
        dec_out.append(torch.empty_like(dec_x[-1]))
        if li % 10 == 9:
            log(f"bench: decode layers resident: {li + 1}")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream

    def step(ev_pre=None, ev_dec=None):
        # events only (no debug outputs): the timed prefill writes nothing but its output
        pre.prefill(xp, outp, events=ev_pre)
        for li in range(n_dec):
            dec_layers[li].decode(dec_x[li], dec_out[li], events=ev_dec[li] if ev_dec else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev_pre = [B.HipEvents(B.MOE_PREFILL_STAGES + 1) for _ in range(K)]
    ev_dec = [[B.HipEvents(B.MOE_DECODE_STAGES + 1) for _ in range(n_dec)] for _ in range(K)]
    marks = B.HipEvents(K + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks.record(0, stream)
    for s in range(K):
        step(ev_pre[s], ev_dec[s])
        marks.record(s + 1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_ms = [marks.elapsed_ms(s, s + 1) for s in range(K)]
    pre_ms = np.array([e.elapsed_ms(0, B.MOE_PREFILL_STAGES) for e in ev_pre])
    stage_all = {name: np.array([e.elapsed_ms(i, i + 1) for e in ev_pre])
                 for i, name in enumerate(B.PREFILL_STAGE_NAMES)}
    stage_ms = {name: float(np.median(v)) for name, v in stage_all.items()}
    prefill_ms = float(np.median(pre_ms))
    tok_s = T / (prefill_ms * 1e-3)

    rows = T * (k + 1)
    gateup_flop = 2.0 * (2 * I) * H * rows
    down_flop = 2.0 * H * I * rows
    router_flop = 2.0 * T * E * H
    gu_ms = stage_ms["gateup"]
    gu_tflops = gateup_flop / (gu_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill {T} tokens (uniform routing) + batch-1 decode over {n_dec} weight sets",
                   "tokens": T, "hidden": H, "experts": E, "top_k": k, "shared_experts": 1, "inter": I,
                   "weights": "int4 affine group-64, fp16 scale/bias", "decode_layers": n_dec},
        "prefill_us": round(prefill_ms * 1e3, 2),
        "prefill_us_p10_p90": [round(pct(pre_ms, 10) * 1e3, 2), round(pct(pre_ms, 90) * 1e3, 2)],
        "prefill_stage_us": {n: round(v * 1e3, 2) for n, v in stage_ms.items()},
        "prefill_tflops": round((gateup_flop + down_flop + router_flop) / (prefill_ms * 1e-3) / 1e12, 1),
        "roofline": {"kernel": "gemm_gateup (grouped GEMM gate/up + SwiGLU)", "bound": "mfma",
                     "achieved": round(gu_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("k_gemm_gateup"), "traffic_unit": "bytes per launch",
                     "algorithmic_flop_per_launch": gateup_flop,
                     "us_p10_p90": [round(pct(stage_all["gateup"], 10) * 1e3, 2),
                                    round(pct(stage_all["gateup"], 90) * 1e3, 2)]},
        "down_roofline": {"kernel": "gemm_down (grouped GEMM down + gate)", "bound": "mfma",
                          "achieved": round(down_flop / (stage_ms["down"] * 1e-3) / 1e12, 1),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(down_flop / (stage_ms["down"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "algorithmic_flop_per_launch": down_flop},
        "step_ms_events": round(float(np.mean(step_ms)), 4),
    }
    if n_dec:
        dec_stage = {name: float(np.median([e.elapsed_ms(i, i + 1) for es in ev_dec for e in es]))
                     for i, name in enumerate(B.DECODE_STAGE_NAMES)}
        dec_layer_ms = float(np.median([e.elapsed_ms(0, B.MOE_DECODE_STAGES) for es in ev_dec for e in es]))
        sweep_ms = np.array([m - p for m, p in zip(step_ms, pre_ms)])
        us_layer = float(np.median(sweep_ms)) * 1e3 / n_dec
        qmat_gu = I * H // 2 + 2 * 2 * I * (H // 64)
        qmat_dn = H * I // 2 + 2 * 2 * H * (I // 64)
        layer_bytes = (k + 1) * (2 * qmat_gu + qmat_dn) + E * H * 2 + 2 * H * 2
        result["decode_us_per_layer"] = round(us_layer, 3)
        result["decode_stage_us"] = {n: round(v * 1e3, 3) for n, v in dec_stage.items()}
        result["decode_layer_us_events"] = round(dec_layer_ms * 1e3, 3)
        result["decode_hbm_frac"] = round(layer_bytes / (us_layer * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        result["decode_algorithmic_bytes_per_layer"] = layer_bytes

    def decode_roofline(us, timing):
        k_gbs = layer_bytes / (us * 1e-6) / 1e9
        return {"kernel": "k_decode (whole decode layer: router, top-k, 9 expert GEMVs)",
                "bound": "hbm", "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(k_gbs / PEAK_HBM_GBS, 4), "timing": timing,
                "traffic": profiled_traffic("k_decode1"), "traffic_unit": "bytes per launch",
                "algorithmic_bytes_per_launch": layer_bytes}

    if n_dec:
        result["decode_roofline"] = decode_roofline(dec_stage["layer"] * 1e3, "HIP events around each call")

    if not args.no_skewed:
        # the skewed workload: the same weights and tokens, router bias with Zipf(1.2)
        # popularity (hot experts of 1000+ rows, about 150 empty)
        log("bench: skewed-routing prefill")
        Ls = synth.make_layer(3)
        sk = MoeLayer(Ls, top_k=k, max_chunk_tokens=T, device=dev)
        del Ls
        _, dsk = sk.prefill(xp, outp, debug=True)
        torch.cuda.synchronize()
        cnt_s = dsk["counts"].cpu().numpy()[0]
        _, dun = pre.prefill(xp, outp, debug=True)
        torch.cuda.synchronize()
        cnt_u = dun["counts"].cpu().numpy()[0]
        ev_s = [B.HipEvents(B.MOE_PREFILL_STAGES + 1) for _ in range(K)]
        for _ in range(args.warmup):
            sk.prefill(xp, outp)
        for s in range(K):
            sk.prefill(xp, outp, events=ev_s[s])
        torch.cuda.synchronize()
        sk_ms = np.array([e.elapsed_ms(0, B.MOE_PREFILL_STAGES) for e in ev_s])
        sk_stage = {name: round(float(np.median([e.elapsed_ms(i, i + 1) for e in ev_s])) * 1e3, 2)
                    for i, name in enumerate(B.PREFILL_STAGE_NAMES)}

        def row_eff(c):
            r, tr = mblock_rows(c)
            return round(float(r.sum() / tr.sum()), 4), int(r.size)

        eff_s, nmb_s = row_eff(cnt_s)
        eff_u, nmb_u = row_eff(cnt_u)
        sk_us = float(np.median(sk_ms)) * 1e3
        result["skewed_prefill"] = {
            "tokens": T, "us": round(sk_us, 2),
            "us_p10_p90": [round(pct(sk_ms, 10) * 1e3, 2), round(pct(sk_ms, 90) * 1e3, 2)],
            "tokens_per_s": round(T / (sk_us * 1e-6), 1), "vs_uniform": round(prefill_ms * 1e3 / sk_us, 4),
            "stage_us": sk_stage, "max_expert_rows": int(cnt_s[:E].max()), "empty_experts": int((cnt_s[:E] == 0).sum()),
            "mfma_row_efficiency": eff_s, "mblocks": nmb_s,
            "uniform_mfma_row_efficiency": eff_u, "uniform_mblocks": nmb_u,
            "gateup_frac": round(gateup_flop / (sk_stage["gateup"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        sk.close()
        del sk, dsk, dun

    if not args.no_ablations:
        # the pages' ablations on this chip: each optimisation switched off alone, prefill
        # of the same layer and tokens at 512 tokens (the pages' prompt for the dequant and
        # routing ablations) and at 4096
        log("bench: ablations")
        variants = {"fixed_32_row_tiles": B.MOE_F_FORCE_BM(32), "host_synced_routing": B.MOE_F_HOST_ROUTING,
                    "separate_dequant": B.MOE_F_SEPARATE_DEQUANT, "no_binary64_rerank": B.MOE_F_NO_FALLBACK}
        abl = {}
        for Tn in (512, T):
            xs = xp[:Tn].contiguous()
            os_ = torch.empty_like(xs)
            base_layer = pre
            runs = {"default": base_layer}
            for name, fl in variants.items():
                runs[name] = pre.with_flags(fl)
            res = {}
            for name, lay in runs.items():
                for _ in range(2):
                    lay.prefill(xs, os_)
                ms = time_events(lambda lay=lay: lay.prefill(xs, os_), max(K // 2, 5), stream, B)
                res[name] = float(np.median(ms)) * 1e3
            abl[str(Tn)] = {name: {"us": round(v, 2), "default_speedup": round(v / res["default"], 4)}
                            for name, v in res.items()}
            for name, lay in runs.items():
                if lay is not base_layer:
                    lay.close()
            del runs
        result["ablations"] = abl

    if not args.no_long_prompt:
        # long prompt (131072 tokens, the same layer) through the chunk driver: one bounded
        # workspace (fixed by the 4096-token chunk), so peak temporary memory is that
        # workspace; torch's allocator is checked for anything beyond it
        shl = synth.shape_of(4)
        log(f"bench: long prompt {shl.T} tokens (drawing x)")
        xl = bf16_tensor(synth.make_x(4), dev)
        outl = torch.empty_like(xl)
        pre.prefill(xl, outl)
        torch.cuda.synchronize()
        base_alloc = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        lmarks = B.HipEvents(3)
        lmarks.record(0, stream)
        pre.prefill(xl, outl)
        lmarks.record(1, stream)
        pre.prefill(xl, outl)
        lmarks.record(2, stream)
        torch.cuda.synchronize()
        l_ms = min(lmarks.elapsed_ms(0, 1), lmarks.elapsed_ms(1, 2))
        extra = int(torch.cuda.max_memory_allocated(dev) - base_alloc)
        result["long_prompt"] = {"tokens": shl.T, "chunk": shl.chunk, "us": round(l_ms * 1e3, 1),
                                 "tokens_per_s": round(shl.T / (l_ms * 1e-3), 1),
                                 "vs_4k_prefill": round(shl.T / (l_ms * 1e-3) / tok_s, 4),
                                 "workspace_bytes": int(pre.ws_bytes), "extra_device_bytes_during_call": extra}
        del xl, outl

    if n_dec and not args.no_graph:
        # the same 40 decode calls captured once in a HIP graph and replayed (their launch
        # arguments do not change between calls), as a serving loop would run them
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for li in range(n_dec):
                dec_layers[li].decode(dec_x[li], dec_out[li])
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        g_ms = time_events(graph.replay, K, stream, B)
        result["decode_us_per_layer_graph"] = round(float(np.median(g_ms)) * 1e3 / n_dec, 3)
        result["decode_us_per_layer_graph_p10_p90"] = [round(pct(g_ms, 10) * 1e3 / n_dec, 3),
                                                       round(pct(g_ms, 90) * 1e3 / n_dec, 3)]
        # back-to-back launches: the per-launch time the kernel trace reports
        result["decode_roofline"] = decode_roofline(result["decode_us_per_layer_graph"],
                                                    f"graph replay of {n_dec} calls, HIP events on the stream")
        del graph

    if n_dec and not args.no_graph:
        # small-batch decode (T rows per call, e.g. a speculative decoder's verification
        # batch): the same 40 weight sets, T rows each, captured once and replayed; the
        # bytes a call must read are the union of the rows' experts (each read once)
        qmat_gu = I * H // 2 + 2 * 2 * I * (H // 64)
        qmat_dn = H * I // 2 + 2 * 2 * H * (I // 64)
        expert_bytes = 2 * qmat_gu + qmat_dn
        batch = {}
        for Tb in (2, 4, 8):
            xb = [torch.stack([dec_x[(li + j) % n_dec] for j in range(Tb)]) for li in range(n_dec)]
            ob = [torch.empty_like(v) for v in xb]
            union = []
            for li in range(n_dec):
                _, d = dec_layers[li].decode_batch(xb[li], ob[li], debug=True)
                union.append(len(set(d["topk_ids"].cpu().numpy().ravel().tolist())) + 1)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for li in range(n_dec):
                    dec_layers[li].decode_batch(xb[li], ob[li])
            g.replay()
            b_ms = time_events(g.replay, K, stream, B)
            us = float(np.median(b_ms)) * 1e3 / n_dec
            nbytes = float(np.mean(union)) * expert_bytes + E * H * 2 + 2 * Tb * H * 2
            batch[str(Tb)] = {"us_per_call": round(us, 3), "us_per_row": round(us / Tb, 3),
                              "active_experts": round(float(np.mean(union)), 2),
                              "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            del g, xb, ob
        result["decode_batch"] = batch

    if not args.no_gdn:
        # the Gated DeltaNet prefill scan of the pages' 2K-token prompt (one layer: 16 key
        # and 32 value heads of width 128), state resident in registers.  Algorithmic work:
        # 3 fmas per state element per token (the dots with k and q, the rank-one update),
        # 6 flops; peak: the vector fp32 fma rate without packed math (this library is
        # built without packed-fp32 instructions): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x
        # 2.4 GHz = 78.6 TFLOP/s (157.3 with packed math)
        from sparse_moe_02_amd.gdn import gdn_scan

        log("bench: gated deltanet scan")
        gs = synth.GDN_CONFIGS[1]
        gi = synth.gdn_inputs(1, seed=0, nonzero_state=True)

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        gq, gk, gv = bf(gi.q), bf(gi.k), bf(gi.v)
        ga, gb = torch.from_numpy(gi.alpha).to(dev), torch.from_numpy(gi.beta).to(dev)
        gst = torch.from_numpy(gi.state).to(dev)
        gout = torch.empty((gs.T, gs.n_vheads, gs.d), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            gdn_scan(gq, gk, gv, ga, gb, gst, gout, stream)
        g_ms = time_events(lambda: gdn_scan(gq, gk, gv, ga, gb, gst, gout, stream), max(K, 10), stream, B)
        g_us = float(np.median(g_ms)) * 1e3
        flop = 6.0 * gs.T * gs.n_vheads * gs.d * gs.d
        gbytes = (gi.q.nbytes + gi.k.nbytes + gi.v.nbytes + gi.alpha.nbytes + gi.beta.nbytes + 2 * gi.state.nbytes
                  + gs.T * gs.n_vheads * gs.d * 2)
        peak_alu = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
        gres = {"workload": f"gdn-2k: {gs.T} tokens, {gs.n_kheads} key / {gs.n_vheads} value heads of {gs.d}",
                "us": round(g_us, 2), "us_p10_p90": [round(pct(g_ms, 10) * 1e3, 2), round(pct(g_ms, 90) * 1e3, 2)],
                "tokens_per_s": round(gs.T / (g_us * 1e-6), 1),
                "roofline": {"bound": "alu", "achieved": round(flop / (g_us * 1e-6) / 1e12, 3),
                             "peak": round(peak_alu, 1), "unit": "TFLOP/s",
                             "frac": round(flop / (g_us * 1e-6) / 1e12 / peak_alu, 4),
                             "frac_vs_packed_peak": round(flop / (g_us * 1e-6) / 1e12 / 157.3, 4),
                             "hbm_bytes": int(gbytes),
                             "hbm_frac": round(gbytes / (g_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}}
        if not args.no_cpu_baseline:
            import oracle

            t1 = time.perf_counter()
            oracle.gdn_scan(gi.q, gi.k, gi.v, gi.alpha, gi.beta, gi.state)
            dt = time.perf_counter() - t1
            gres["cpu_baseline"] = {"value": round(gs.T / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                    "sample": f"the full {gs.T}-token scan ({dt:.2f} s)"}
        result["gdn_scan"] = gres
        del gq, gk, gv, ga, gb, gst, gout

    if not args.no_ceilings:
        log("bench: measured ceilings")
        c = ceilings(dev, stream, B, dec_layers, dec_x, H, I, k)
        result["ceilings"] = c
        result["roofline"]["frac_vs_measured"] = round(gu_tflops / c["mfma_bf16_TFLOPs"], 4)
        result["roofline"]["measured_peak"] = c["mfma_bf16_TFLOPs"]
        result["roofline"]["frac_vs_random_data_mfma"] = round(gu_tflops / c["mfma_bf16_random_data_TFLOPs"], 4)
        result["roofline"]["frac_vs_dequant_pipeline"] = round(gu_tflops / c["dequant_mfma_pipeline_TFLOPs"], 4)
        if "decode_roofline" in result:
            dr = result["decode_roofline"]
            dr["frac_vs_measured"] = round(dr["achieved"] / c["hbm_read_GBs"], 4)
            dr["measured_peak"] = c["hbm_read_GBs"]
            if "layer_bytes_flat_stream_us" in c and "decode_us_per_layer_graph" in result:
                # the single-phase read of the same bytes, routing given: the floor this
                # dependency chain (router -> selection -> gate/up -> down) sits above
                dr["frac_vs_flat_stream"] = round(c["layer_bytes_flat_stream_us"] / result["decode_us_per_layer_graph"],
                                                  4)

    if not args.no_cpu_baseline:
        import oracle

        log("bench: oracle CPU baseline (full 4096-token prefill of the same layer)")
        t1 = time.perf_counter()
        oracle.forward(xp_bits, Lp, k)
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(T / dt, 2), "unit": "tokens/s", "cores": oracle.threads(),
                                  "kind": "oracle",
                                  "sample": f"the full {T}-token prefill of the benchmark layer ({dt:.1f} s)"}
    print(json.dumps(result), flush=True)
    for layer in dec_layers + [pre]:
        layer.close()


if __name__ == "__main__":
    main()
