#!/usr/bin/env python3
"""Throughput of the CSA2 hot path on one MI355X, with roofline and CPU-oracle baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--topk-route auto|scores|score-free] [--flush auto|on|off] [--graph] [--calibrate]

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM:
  decode  : indexer_score -> topk_select -> sparse_attn_decode
            (wide FULL rows with an FP8 or MXFP4 index plane keep their scores on chip:
            indexer_score(scores=None) -> topk_rescore; a FULL owner layer that
            builds the REINDEX candidate pool adds candidate_pool from the block
            scores the indexer wrote)
  prefill : indexer_score -> topk_select -> sparse_attn_prefill for the FULL
            layer and every REUSE layer (same indices, own q / SWA / sink);
            --topk-route score-free takes the chunk's score-free route instead
            (block keys, the best blocks re-scored, exact select)
The default workload is the 1M-context low-precision decode (64 sequences,
FP8 index plane, FP4 main plane, FP8 SWA ring).  Prints one JSON line.

After the warmup, a pass of K steps with HIP events around every call gives
the per-call times and the dominant call; then the K timed steps carry events
around the dominant call only (each event costs the stream a few
microseconds), which give the roofline's kernel time.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn query-tokens/s + achieved HBM GB/s, decode at 1M context, 1 MI355X"
# Workloads whose bytes (157-289 MiB) are about the size of the 256 MB last-level cache (MALL): reading a
# 512 MiB buffer between timed steps evicts their planes, so each step reads them from HBM.  (A read, not a
# write: a write leaves ~256 MB of dirty lines whose write-back would land inside the next step's kernels.)
FLUSH_DEFAULT = {"full_decode_64k", "reindex_decode_1m", "reindex_fp8_decode_1m", "reindex_pages_decode_1m"}
FLUSH_BYTES = 512 << 20
HBM_PEAK_GBS = 8000.0
DEFAULT_CONFIG = "lowp_full_decode_1m"

_ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


# Dense matrix-core peaks of MI355X by operand type (TFLOP/s, no sparsity).
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0, "f32": 157.3}


def _row_bytes(dtype, d):
    """Stored bytes of one d-element row, scales included."""
    return {"f32": 4 * d, "bf16": 2 * d, "fp8": d + 4, "fp4": d // 2 + d // 32, "nvfp4": d // 2 + d // 16,
            "fp8mx": d + d // 32}[dtype]


def _unique_plane_rows(base, rows_read):
    """Distinct plane rows over query rows: rows_read(r) -> local row ids of row r, offset by its plane base."""
    import torch
    seen = [base[r] + rows_read(r) for r in range(base.shape[0])]
    return int(torch.unique(torch.cat(seen)).numel()) if seen else 0


def algorithmic_work(cfg, x, idx_host=None, score_free=False, bk_bytes=4):
    """Per kernel of one step: the bytes it must move at least once (every distinct input byte read
    once, every output byte written once) and the multiply-add flops it must do.

    Queries that share one plane (a prefill chunk) read each distinct plane row once; decode rows
    each own a plane.  Flops count 2 per multiply-add: the indexer's 64 x 128 head dots per scored
    column, attention's QK^T and PV (2 x H x D multiply-adds per entry row per query)."""
    import torch
    pos = x["pos"].cpu()
    base = x["kv_row_base"].cpu()
    nv = ((pos + 1) // cfg.ratio).clamp(max=cfg.n_main_rows)
    rows = pos.shape[0]
    idx_row = _row_bytes(cfg.idx_dtype, cfg.idx_dim)
    # the query (FP8: no scale, it is folded into w) and the head weights
    q_row = cfg.idx_dim if cfg.idx_dtype == "fp8" else _row_bytes(cfg.idx_dtype, cfg.idx_dim)
    qI = rows * cfg.idx_heads * q_row + rows * cfg.idx_heads * 4
    if cfg.index_mode == "reindex":
        cand = x["cand"].cpu().long()
        cols = cand.repeat_interleave(cfg.block_rows, dim=1) * cfg.block_rows + \
            torch.arange(cfg.block_rows).repeat(cfg.n_blocks)
        valid = (cand.repeat_interleave(cfg.block_rows, dim=1) >= 0) & (cols < nv[:, None])
        scored = int(valid.sum())
        unique_rows = _unique_plane_rows(base, lambda r: cols[r][valid[r]])
        extra = rows * cfg.n_blocks * 4
    else:
        scored = int(nv.sum())
        unique_rows = sum(int(nv[base == b].max()) for b in torch.unique(base))
        extra = 0
    nbm = -(-cfg.width // cfg.block_rows) if cfg.pool_blocks else 0
    if score_free:
        # scores stay on chip: only the 8-column block keys are written (bk_bytes each: 4, or 2 when
        # only their top 16 bits are kept)
        nbk = -(-cfg.width // 8)
        idx_bytes = unique_rows * idx_row + qI + rows * nbk * bk_bytes
        nbm = nbk if cfg.pool_blocks else 0  # the pool ranks the same block keys
        # the select reads the block keys (re-scored candidate rows and the second look at the block
        # keys are not counted: they are extra work of this route, not bytes the result needs)
        topk_bytes = rows * nbk * bk_bytes + rows * cfg.topk * 4
    else:
        idx_bytes = unique_rows * idx_row + qI + extra + rows * cfg.width * 4 + rows * nbm * 4
        topk_bytes = rows * cfg.width * 4 + rows * cfg.topk * 4 + extra
    idx_flops = 2 * scored * cfg.idx_heads * cfg.idx_dim
    main_row = _row_bytes(cfg.main_dtype, cfg.dim)
    swa_row = _row_bytes(cfg.swa_dtype, cfg.dim)
    sel = torch.minimum(nv, torch.tensor(cfg.topk))
    win = torch.minimum(pos + 1, torch.tensor(cfg.window))
    layers = len(x["layers"])
    qo = rows * cfg.heads * cfg.dim * (_ELEM[cfg.q_dtype] + _ELEM[cfg.out_dtype])
    if cfg.phase == "decode":
        main_rows, swa_rows = int(sel.sum()), int(win.sum())
    else:
        # one chunk: distinct selected rows of the shared plane, and the linear SWA array once
        ii = idx_host
        main_rows = int(torch.unique(ii[ii >= 0]).numel()) if ii is not None else int(sel.sum())
        swa_rows = int(pos.max() - pos.min()) + cfg.window
    # one launch per layer; each re-reads the selected rows and its own q / SWA
    attn_bytes = layers * (main_rows * main_row + swa_rows * swa_row + qo + rows * cfg.topk * 4)
    attn_flops = layers * 4 * cfg.heads * cfg.dim * int((sel + win).sum())
    attn_dt = "f32" if cfg.q_dtype == "f32" else "bf16"
    # candidate pool: read the block scores, write the kept blocks
    pool_bytes = rows * nbm * 4 + rows * cfg.pool_blocks * 4
    # write path (owner layers): the hidden rows and the weights once, the new rows of both planes, the
    # tail state; flops of the projections (kv [+ gate]) and of the index-key projection of each new row
    comp = (0, 0, None, 1)
    if cfg.d_model:
        nproj = 512 * cfg.ratio
        emitted = rows if cfg.ratio == 1 else int((pos % 2 == 1).sum())
        comp_bytes = (rows * cfg.d_model * 2 + nproj * cfg.d_model * 2 + 128 * 512 * 2 + (512 + 128) * 4
                      + emitted * (main_row + idx_row) + rows * 8 * 2 + (rows * 512 * 8 if cfg.ratio == 2 else 0))
        comp = (comp_bytes, 2 * rows * cfg.d_model * nproj + 2 * emitted * 512 * 128, "bf16", 1)
    return {"compress": comp,
            "indexer_score": (idx_bytes, idx_flops, cfg.idx_dtype, 1),
            "topk_select": (topk_bytes, 0, None, 1),
            "candidate_pool": (pool_bytes, 0, None, 1),
            "sparse_attn": (attn_bytes, attn_flops, attn_dt, layers),
            "scored_rows": scored}


def roofline_of(work, ms):
    """Bound (the HBM or matrix-core roof the kernel's intensity puts it under), achieved and fraction."""
    nbytes, flops, dt, _ = work
    t = ms * 1e-3
    if dt is not None and flops > 0:
        peak_flops = MFMA_PEAK_TFLOPS[dt] * 1e12
        if flops / nbytes > peak_flops / (HBM_PEAK_GBS * 1e9):
            achieved = flops / t / 1e12
            return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS[dt],
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS[dt], 4)}
    achieved = nbytes / t / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}


KERNEL_SOURCES = {
    "indexer_score": ["indexer.hip", "common.hpp", "kernels.hpp"],
    "topk_select": ["topk.hip", "indexer.hip", "common.hpp", "kernels.hpp"],  # the score-free select re-scores
    "candidate_pool": ["topk.hip", "pool.hip", "common.hpp", "kernels.hpp"],
    "compress": ["compress.hip", "common.hpp", "kernels.hpp"],
    "sparse_attn": ["attention.hip", "common.hpp", "kernels.hpp"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "sparse_latent_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was
    taken on the current sources of this kernel (profiles/traffic_<workload>.md, json block)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)["kernels"].get(kernel)
    except (IndexError, ValueError, KeyError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return int(round((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024))


def cpu_baseline(cfg, x, budget_s=20.0):
    """The oracle (float64 NumPy) on the host, one query row at a time, for about budget_s seconds."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_info
    tests_dir = os.path.join(ROOT, "tests")
    sys.path.insert(0, tests_dir)
    from harness import oracle_attention, oracle_scores, oracle_topk  # noqa: E402
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    done, t_total = 0, 0.0
    rows = x["pos"].shape[0]
    for r in range(rows):
        # Copy this row's inputs to the host before timing (not part of the oracle's work).
        sub = _host_slice(cfg, x, r)
        sub_cfg = cfg.replace(batch=1, q_tokens=1)
        t0 = time.perf_counter()
        if cfg.d_model:
            oracle.compressor.compress_call(*sub["compress_args"])
        s = oracle_scores(sub_cfg, sub, np.array([0]))
        idx = oracle_topk(sub_cfg, sub, s, np.array([0]))
        if cfg.pool_blocks:
            oracle.candidates.candidate_pool(s, sub["pos"].numpy(), cfg.ratio, cfg.block_rows, cfg.pool_blocks)
        for layer in range(len(sub["layers"])):
            oracle_attention(sub_cfg, sub, idx, np.array([0]), layer=layer)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    return {"value": done / t_total, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {rows} query rows of the {cfg.name} batch, whole path ("
                      f"{'write path of the row, ' if cfg.d_model else ''}indexer, top-k, "
                      f"{'candidate pool, ' if cfg.pool_blocks else ''}attention"
                      f"{' x %d layers' % len(x['layers']) if len(x['layers']) > 1 else ''}), float64 NumPy; "
                      f"host copy excluded; {t_total:.1f} s"}


def oracle_rope_freqs(cfg):
    import oracle
    return oracle.rope.inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig)


def _host_slice(cfg, x, r):
    """Inputs of query row r alone, on the host (decode: its sequence; prefill: the shared planes)."""
    import numpy as np
    import torch
    out = {"cfg": cfg}
    cpu = lambda t: None if t is None else t.detach().cpu()
    if cfg.phase == "decode":
        b = r
        out["pos"] = cpu(x["pos"][b:b + 1])
        out["kv_row_base"] = torch.zeros(1, dtype=torch.int64)
        out["main"] = cpu(x["main"][b:b + 1])
        out["main_scale"] = cpu(None if x["main_scale"] is None else x["main_scale"][b:b + 1])
        out["kI"] = cpu(x["kI"][b:b + 1])
        out["kI_scale"] = cpu(None if x["kI_scale"] is None else x["kI_scale"][b:b + 1])
        out["swa"] = cpu(x["swa"][b:b + 1])
        out["swa_scale"] = cpu(None if x["swa_scale"] is None else x["swa_scale"][b:b + 1])
        out["layers"] = [{"q": cpu(L["q"][b:b + 1]), "sink": cpu(L["sink"])} for L in x["layers"]]
    else:
        out["pos"] = cpu(x["pos"][r:r + 1])
        out["kv_row_base"] = torch.zeros(1, dtype=torch.int64)
        out["main"], out["main_scale"] = cpu(x["main"]), cpu(x["main_scale"])
        out["kI"], out["kI_scale"] = cpu(x["kI"]), cpu(x["kI_scale"])
        out["swa_pos0"] = x["swa_pos0"]
        out["layers"] = [{"q": cpu(L["q"][r:r + 1]), "swa": cpu(L["swa"]), "swa_scale": cpu(L["swa_scale"]),
                          "sink": cpu(L["sink"])} for L in x["layers"]]
    if cfg.d_model:
        # the write path's work for this row's token (with its group partner at ratio 2), float64 host arrays
        c = x["compress"]
        f64 = lambda t: None if t is None else t.detach().cpu().double().numpy()
        rs = [r - 1, r] if cfg.ratio == 2 and r > 0 and int(c["pos"][r]) % 2 == 1 else [r]
        freqs = oracle_rope_freqs(cfg)
        out["compress_args"] = (f64(c["x"][rs]), c["pos"][rs].cpu().numpy(), np.zeros(len(rs), dtype=np.int64),
                                cfg.ratio, f64(c["wkv"]), f64(c["wgate"]), f64(c["norm_w"]), 1e-6, f64(c["wk"]),
                                f64(c["knorm_w"]), 1e-6, freqs, None if c["tail_kv"] is None else f64(c["tail_kv"][:1]),
                                None if c["tail_score"] is None else f64(c["tail_score"][:1]))
    out["qI"] = cpu(x["qI"][r:r + 1])
    out["qI_scale"] = cpu(None if x.get("qI_scale") is None else x["qI_scale"][r:r + 1])
    out["w"] = cpu(x["w"][r:r + 1])
    if "cand" in x:
        out["cand"] = cpu(x["cand"][r:r + 1])
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--flush", choices=["auto", "on", "off"], default="auto",
                    help="read 512 MiB between timed steps (outside the timed events) so the planes come from HBM; "
                         "auto: on for the workloads about the size of the MALL (64K decode, 1M REINDEX decodes)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the same step captured once in a HIP graph and replayed (reported under "
                         "\"graph\"; value stays the eager launches)")
    ap.add_argument("--topk-route", choices=["auto", "scores", "score-free"], default="auto",
                    help="how the FULL layer's top-k is found: auto (score-free for wide FP8/MXFP4 rows, written "
                         "scores otherwise), scores (write the score rows, then topk_select) or score-free (block "
                         "keys only, then topk_rescore; the prefill chunk's BF16 rows take it only when asked)")
    ap.add_argument("--calibrate", action="store_true",
                    help="after the bench, run a plain 1 GiB float32 copy kernel 3 times (the reference for "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE scaling: 1 GiB read + 1 GiB written per launch)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              f"sequence with no communication, so N GPUs would each run this same workload.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import CONFIGS, make_inputs
    from workloads.step import Step

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} seed {args.seed}", file=sys.stderr, flush=True)
    x = make_inputs(cfg, args.seed, device=dev)
    torch.cuda.synchronize()

    rows = x["pos"].shape[0]
    # Arguments are marshalled once; each step only crosses into the library.
    route = {"auto": None, "scores": False, "score-free": True}[args.topk_route]
    step_calls = Step(cfg, x, score_free=route)
    names = list(step_calls.groups)
    flush = args.flush == "on" or (args.flush == "auto" and cfg.name in FLUSH_DEFAULT)
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if flush else None

    def run_steps(n, bracket):
        """n steps; events around every group in `bracket` (recording an event costs the stream about
        5 us, so the timed steps bracket the dominant group only).  Returns per-group event pairs and,
        with the flush, each step's own event pair."""
        evs = {g: [] for g in bracket}
        step_evs = []

        def event():
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            return e

        for _ in range(n):
            a = None
            if flush:
                flush_buf.sum()  # evicts the planes (a 512 MiB read); outside the step's events
                a = event()
            state = {"open": None, "first": True, "end": None}

            def on_group(name):
                # name None: the step's end.  The step's own start and end events serve a first or
                # last bracketed group.
                if state["open"] is not None:
                    g, e0 = state["open"]
                    e1 = event()
                    evs[g].append((e0, e1))
                    state["open"] = None
                    if name is None:
                        state["end"] = e1
                if name in bracket:
                    state["open"] = (name, a if (state["first"] and a is not None) else event())
                state["first"] = False

            step_calls(on_group)
            if flush:
                step_evs.append((a, state["end"] if state["end"] is not None else event()))
        return evs, step_evs

    def mean_ms(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    run_steps(args.warmup, ())
    torch.cuda.synchronize()
    # Pass 1 (not the timed steps): every group bracketed, for the per-call times and the dominant call.
    print(f"[bench] per-call pass {args.steps} steps", file=sys.stderr, flush=True)
    evs, _ = run_steps(args.steps, set(names))
    torch.cuda.synchronize()
    kern_ms = {n: mean_ms(evs[n]) for n in names}
    dominant = max(names, key=lambda n: kern_ms[n])
    # Pass 2, the timed steps: events around the dominant call only.
    print(f"[bench] timing {args.steps} steps{' (L2/MALL flushed between steps)' if flush else ''}",
          file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs_t, step_evs = run_steps(args.steps, {dominant})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if flush:
        # with a flush between steps the wall clock includes it: the step time is the events' span
        ms_step = mean_ms(step_evs)
    else:
        ms_step = wall * 1e3 / args.steps
    dom_ms = mean_ms(evs_t[dominant])

    bk = step_calls.block_keys
    work = algorithmic_work(cfg, x, step_calls.idx.cpu() if cfg.phase == "prefill" else None, step_calls.score_free,
                            4 if bk is None else bk.element_size())
    roofline = roofline_of(work[dominant], dom_ms)
    roofline.update({"kernel": dominant, "traffic": measured_traffic(dominant, cfg.name),
                     "launches_per_step": work[dominant][3],
                     "algorithmic_bytes_per_launch": work[dominant][0] // work[dominant][3],
                     "algorithmic_flops_per_launch": work[dominant][1] // work[dominant][3],
                     "source_hash": kernel_source_hash(dominant)})
    q_tokens = rows
    line = {
        "metric": METRIC, "value": round(q_tokens / (ms_step * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp4": "fp4+bf16", "fp8": "fp8+bf16", "bf16": "bf16", "f32": "f32"}[cfg.idx_dtype],
        "data": "synthetic (seeded; stored formats drawn as in workloads/gen.py)",
        "config": {"workload": cfg.name, "sequences": cfg.batch, "query_rows": rows, "context": cfg.context,
                   "ratio": cfg.ratio, "heads": cfg.heads, "dim": cfg.dim, "topk": cfg.topk, "window": cfg.window,
                   "index": f"{cfg.index_mode} {cfg.idx_heads}x{cfg.idx_dim} {cfg.idx_dtype}",
                   "main_kv": cfg.main_dtype, "swa": cfg.swa_dtype, "attention_layers": len(x["layers"]),
                   "topk_route": "score-free (topk_rescore)" if step_calls.score_free else "scores + topk_select",
                   "write_path": f"d_in {cfg.d_model}, ratio {cfg.ratio}" if cfg.d_model else None},
        "timing": (("HIP events around each step; 512 MiB read between steps (L2/MALL flush, not timed); "
                    f"wall clock incl. flush {wall * 1e3 / args.steps:.4f} ms/step") if flush else
                   "wall clock over the timed steps (synchronized before and after)") +
                  f"; the timed steps carry HIP events around {dominant} only (roofline); kernels_ms from a "
                  f"separate pass of {args.steps} steps with events around every call",
        "kernels_ms": {n: round(v, 4) for n, v in kern_ms.items()},
        "kernels_roofline": {n: roofline_of(work[n], kern_ms[n]) for n in names},
        "roofline": roofline,
    }
    if args.graph:
        # The step's calls prepared again on a side stream (a graph is captured on one), captured once, and
        # replayed K times: the kernels are the same, the launches come from the graph.
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            g_step = Step(cfg, x, score_free=route)
            g_step()
        gs.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            g_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g_evs = []
        t1 = time.perf_counter()
        for _ in range(args.steps):
            if flush:
                flush_buf.sum()
                a = torch.cuda.Event(enable_timing=True)
                a.record()
            graph.replay()
            if flush:
                b = torch.cuda.Event(enable_timing=True)
                b.record()
                g_evs.append((a, b))
        torch.cuda.synchronize()
        g_wall = time.perf_counter() - t1
        g_ms = mean_ms(g_evs) if flush else g_wall * 1e3 / args.steps
        line["graph"] = {"ms_per_step": round(g_ms, 4), "value": round(q_tokens / (g_ms * 1e-3), 1),
                         "timing": "HIP events around each replay" if flush else "wall clock over the replays"}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_budget)
    print(json.dumps(line), flush=True)
    if args.calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy": {"bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                                               "launches": 3}}), flush=True)


if __name__ == "__main__":
    main()
