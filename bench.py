"""Benchmark of the HSA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config c1_full] [--no-cpu-baseline]

One step = the whole hot path over one chunk of one layer: page scoring ->
gather -> linear branch -> block selection -> sparse branch -> fusion (six
C-ABI calls; the linear branch on a side stream), on seeded synthetic inputs
already resident in HBM.  Prints ONE JSON line.  The metric is ms per chunk
(lower is better); attended TFLOP/s of the sparse branch, per-stage times,
the roofline of the dominant kernel and the CPU oracle's time (bounded
sample) are reported in the same line.

Variants (each reports its own line; the default is the headline workload):
  --config c4_stack        the 30-layer x 4-step chunk with host-resident pages
  --page-index             score from mean keys kept when pages were written
  --chunks K               prompt-level retrieval first (top-K chunks), scoring
                           only their pages (--pages-per-chunk, default 8)
  --tiers N                N generated chunks over a history in page tiers,
                           fetched on demand vs predicted and prefetched
  --paged                  pages laid out once when written; the step scores from
                           the page index and reads the selected pages in place
                           (no active-buffer copy)
  --intra S                the chunk's own tokens join the retrieved history in
                           key blocks of B/S tokens (intra-chunk keys)
  --graph                  the step replayed as one HIP graph
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

METRIC = "HSA ms/chunk at 49,920 retrieved tokens; attended TFLOP/s & % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3      # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
STAGES = ("score", "gather", "linear", "select", "sparse", "fuse")


def stage_model(cfg, n_sel_total: int, indexed: bool = False, scored_pages=None, paged: bool = False):
    """Algorithmic work of one call of each stage (bytes moved or flops).
    With the page index, scoring reads the pages' fp32 mean keys instead of
    their keys; with prompt-level retrieval it reads only scored_pages."""
    es = 2 if cfg.dtype == "bf16" else 4
    H, d, Lp, Lq, L, B, r, P = (cfg.n_heads, cfg.head_dim, cfg.page_tokens, cfg.query_tokens,
                                cfg.active_tokens, cfg.block, cfg.rank,
                                cfg.n_pages if scored_pages is None else scored_pages)
    D = H * d
    Bk, nC = cfg.key_block, cfg.n_candidates  # key-block size; selection candidates per row
    return {
        "score": dict(bound="hbm", bytes=(P * D * 4 if indexed else P * Lp * D * es) + Lq * D * es),
        # paged: the gather stage only moves the selected pages' block means
        # (and with intra-chunk keys lays out the chunk's own keys and values)
        "gather": dict(bound="hbm", bytes=(2 * H * (L // Bk) * d * 4 + (4 * Lq * D * es if cfg.intra_split else 0))
                       if paged else 2 * (2 * L * D * es)),
        "linear": dict(bound="mfma", flops=2 * 2 * H * r * L * d + 2 * 2 * H * Lq * r * d,
                       bytes=2 * L * D * es + 2 * r * L * es + Lq * D * es + Lq * D * 4),
        "select": dict(bound="hbm", bytes=Lq * D * es + H * (L // Bk) * d * 4,
                       flops=2 * H * (Lq // B) * nC * d),
        "sparse": dict(bound="mfma", flops=4 * B * Bk * d * n_sel_total),
        "fuse": dict(bound="hbm", bytes=Lq * D * es + 2 * Lq * D * 4 + Lq * D * es, flops=2 * Lq * D * 2 * H),
    }


def measured_peaks():
    """What this GPU sustains, measured here (the published peaks are the
    roofline's denominators; these are reported beside them): the bf16
    matrix-core rate of a register-only product loop, and the HBM rate of a
    1 GiB stream copy (read + write bytes), both through the library's probe
    entry points.  Best of three runs each."""
    import torch
    from sparse_linear_attention_hsa_amd import ops
    n_wg, iters = 256, 2000
    out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ops.hsa_probe_mfma_bf16(n_wg, iters, out, a, b)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    mfma_tf = n_wg * 8 * iters * 32 * 16 * 16 * 32 * 2 / (best * 1e-3) / 1e12
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    ops.hsa_probe_hbm_copy(x, y, None, None)
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ops.hsa_probe_hbm_copy(x, y, a, b)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x, y
    return {"mfma_bf16_tflops": round(mfma_tf, 1), "hbm_copy_gbs": round(2 * n / (best * 1e-3) / 1e9, 1)}


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when there is none for this workload or the kernel
    source (or the host code that cuts its work items) has changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", f"sparse_attn_kernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from sparse_linear_attention_hsa_amd.profiling import source_digest
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _oracle_pass(cfg, arrays, nh):
    """One timed pass of the float64 oracle over the sample; per-stage seconds."""
    from oracle import hsa_oracle as orc
    s, pk, pv = arrays
    H, B = cfg.n_heads, cfg.block
    intra = bool(cfg.intra_split)
    t = {}
    t0 = time.perf_counter()
    sc = orc.score_and_select(s["q"], pk, cfg.n_sel_pages)
    t["score"] = time.perf_counter() - t0
    sel = sc["sel"]
    t0 = time.perf_counter()
    cat_k = orc.gather_active(pk, sel)
    cat_v = orc.gather_active(pv, sel)
    if intra:  # the chunk's own keys follow the pages
        cat_k = np.concatenate([cat_k, np.asarray(s["k_cur"], np.float64).transpose(1, 0, 2)], axis=1)
        cat_v = np.concatenate([cat_v, np.asarray(s["v_cur"], np.float64).transpose(1, 0, 2)], axis=1)
        parts = orc.key_parts(cfg.history_tokens, B, cfg.query_tokens, cfg.key_block)
    t["gather"] = time.perf_counter() - t0
    q = np.asarray(s["q"], dtype=np.float64)
    t0 = time.perf_counter()
    lin = orc.linear_branch(q, cat_k, cat_v, s["e_k"], s["e_v"])
    t["linear"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    bs = orc.block_selection_parts(q, cat_k, s["tau"], B, parts) if intra else orc.block_selection(q, cat_k, s["tau"], B)
    t["select"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    if intra:
        o_sp = orc.sparse_attention_parts(q[:, :nh], cat_k[:nh], cat_v[:nh], bs["sel"][:nh], B, parts)
    else:
        o_sp = orc.sparse_attention(q[:, :nh], cat_k[:nh], cat_v[:nh], bs["sel"][:nh], B)
    t["sparse"] = (time.perf_counter() - t0) * H / nh
    o_full = np.zeros((cfg.query_tokens, H, cfg.head_dim))
    o_full[:, :nh] = o_sp
    t0 = time.perf_counter()
    orc.fuse(s["x"], s["w_g"], lin["o_lin"], o_full)
    t["fuse"] = time.perf_counter() - t0
    return t


def cpu_baseline(cfg, w, arrays):
    """Time the float64 oracle on a bounded sample of the same workload and
    scale it to one chunk: scoring, gather, linear branch, block selection
    and fusion run whole; the sparse branch runs for the first three heads
    on every query block (x H/3).  The median of three passes with every
    host core, then one pass on one thread (and the tiny workload's whole
    oracle step on one thread)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from synth import C0, Workload
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    nh = min(3, cfg.n_heads)
    runs = [_oracle_pass(cfg, arrays, nh) for _ in range(3)]
    totals = [1e3 * sum(t.values()) for t in runs]
    med = int(np.argsort(totals)[1])
    with threadpool_limits(limits=1):
        one = 1e3 * sum(_oracle_pass(cfg, arrays, nh).values())
        w0 = Workload(C0)
        s0 = w0.small_inputs()
        pk0, pv0 = w0.pages()
        one_c0 = 1e3 * sum(_oracle_pass(C0, (s0, pk0, pv0), C0.n_heads).values())
    return {"value": round(totals[med], 1), "unit": "ms/chunk", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 NumPy oracle; scoring, gather, linear branch, block selection and fusion whole; "
                      f"sparse branch on heads 0..{nh - 1} of {cfg.n_heads}, every query block (x{cfg.n_heads}/{nh}); "
                      f"median of 3 passes on {cores} threads",
            "runs_ms": [round(v, 1) for v in totals],
            "stages_ms": {k: round(1e3 * v, 1) for k, v in runs[med].items()},
            "one_thread_ms": {cfg.name: round(one, 1), C0.name: round(one_c0, 3)}}


def run_stack(args, cfg):
    """A whole chunk of a layer stack (every layer x every denoising step),
    with the configured share of the selected pages starting in pinned host
    memory and streamed in on a side stream.  The same chunk also runs with
    every page resident; the difference is the exposed host-to-device time."""
    import torch
    from synth import layer_arrays, stack_host_pages
    from sparse_linear_attention_hsa_amd.ops import make_geom
    from sparse_linear_attention_hsa_amd.stack import HsaStack, LayerInputs, make_layer_inputs

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    geom = make_geom(cfg.n_heads, cfg.head_dim, cfg.frame_h, cfg.frame_w, cfg.frames_per_page,
                     cfg.query_frames, cfg.tile, cfg.n_sel_pages, cfg.rank, cfg.dtype)
    host_ids = stack_host_pages(cfg)
    up = lambda a: torch.from_numpy(a).to(tdt).cuda()
    streamed, resident = [], []
    for l in range(cfg.layers):
        a = layer_arrays(cfg, l, cfg.steps, workers=16)
        pk = [up(x) for x in a["pages_k"]]
        pv = [up(x) for x in a["pages_v"]]
        qs = [up(x) for x in a["q"]]
        xs = [up(x) for x in a["x"]]
        e_k, e_v, w_g = up(a["e_k"]), up(a["e_v"]), up(a["w_g"])
        tau = torch.from_numpy(a["tau"]).cuda()
        del a
        lay = make_layer_inputs(geom, pk, pv, host_ids[l], e_k, e_v, w_g, tau, qs, xs)
        streamed.append(lay)
        resident.append(LayerInputs(pages_k=pk, pages_v=pv, host_k={}, host_v={}, e_k=e_k, e_v=e_v, w_g=w_g,
                                    tau=tau, page_kmean=lay.page_kmean, q=lay.q, x=lay.x))
        print(f"bench: layer {l + 1}/{cfg.layers} ready ({len(host_ids[l])} host pages)", file=sys.stderr, flush=True)
    max_host = max(len(h) for h in host_ids)
    stack = HsaStack(geom, cfg.n_pages, cfg.layers, max_host)
    stream = torch.cuda.current_stream()

    def timed(inputs, k):
        for _ in range(args.warmup):
            stack.run_chunk(inputs, cfg.steps, {})
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            stack.run_chunk(inputs, cfg.steps, {})
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    ms = timed(streamed, args.steps)
    ms_res = timed(resident, args.steps)
    # the host-to-device copies alone: every non-resident page of the chunk, back to back
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for lay in streamed:
        for n, j in enumerate(sorted(lay.host_k)):
            stack.stage_k[0][n].copy_(lay.host_k[j], non_blocking=True)
            stack.stage_v[0][n].copy_(lay.host_v[j], non_blocking=True)
    b.record(stream)
    torch.cuda.synchronize()
    h2d_ms = a.elapsed_time(b)
    h2d_bytes = sum(2 * cfg.page_tokens * cfg.model_dim * (2 if cfg.dtype == "bf16" else 4) * len(h) for h in host_ids)
    out = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms/chunk", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "denoise_steps": cfg.steps, "heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "retrieved_tokens": cfg.active_tokens,
                   "query_tokens": cfg.query_tokens, "history_pages": cfg.n_pages, "block": cfg.block,
                   "rank": cfg.rank, "host_pages": int(sum(len(h) for h in host_ids))},
        "ms_per_layer_step": round(ms / (cfg.layers * cfg.steps), 4),
        "ms_all_resident": round(ms_res, 3),
        "exposed_h2d_ms": round(ms - ms_res, 3),
        "h2d_bytes": int(h2d_bytes),
        "h2d_ms_alone": round(h2d_ms, 3),
        "h2d_gbs": round(h2d_bytes / (h2d_ms * 1e-3) / 1e9, 1),
        "staging_slots": stack.n_slots,
    }
    print(json.dumps(out), flush=True)


def run_tiers(args, cfg):
    """Several generated chunks over one history whose pages live in tiers
    (device slots for one chunk's K_p pages, pinned host slots for half the
    history, the full backup in pageable host memory).  Per chunk: stage 1
    and chunk-restricted scoring from the page index, the selected pages made
    resident, the gather, then the per-step stages repeated R times (a
    stand-in for the layers and denoising steps of one chunk).  Two runs:
    pages fetched when selected, and the next chunk's pages predicted by
    stage 1 on its prompt and prefetched during the current chunk."""
    import torch
    from synth import Workload, chunk_prompt_sequence
    from sparse_linear_attention_hsa_amd import ops
    from sparse_linear_attention_hsa_amd.ops import make_geom
    from sparse_linear_attention_hsa_amd.step import HsaStep
    from sparse_linear_attention_hsa_amd.tiers import PageTiers

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    kp, n_chunks_gen, R = cfg.n_sel_pages, args.tiers, args.tiers_steps
    w = Workload(cfg)
    s = w.small_inputs()
    up = lambda a: torch.from_numpy(a).to(tdt).cuda()
    q, x, e_k, e_v, w_g = (up(s[k]) for k in ("q", "x", "e_k", "e_v", "w_g"))
    k_cur, v_cur = (up(s["k_cur"]), up(s["v_cur"])) if cfg.intra_split else (None, None)
    tau = torch.from_numpy(s["tau"]).cuda()
    pk_np, pv_np = w.pages()
    geom = make_geom(cfg.n_heads, cfg.head_dim, cfg.frame_h, cfg.frame_w, cfg.frames_per_page,
                     cfg.query_frames, cfg.tile, cfg.n_sel_pages, cfg.rank, cfg.dtype)
    page_chunk, prompts, prev, targets = chunk_prompt_sequence(cfg, kp, n_chunks_gen)
    pc_d, prev_d = torch.from_numpy(page_chunk).cuda(), torch.from_numpy(prev).cuda()
    prompts_d = [torch.from_numpy(p).cuda() for p in prompts]
    n_hist = len(prev)

    def run(prefetch: bool):
        st = HsaStep(geom, cfg.n_pages)
        # the page index, built when the pages were written
        st.index_pages(q, [up(p) for p in pk_np])
        torch.cuda.synchronize()
        tiers = PageTiers(pk_np, pv_np, l1_slots=kp, l2_slots=cfg.n_pages // 2, dtype=tdt,
                          l2_pages=range(cfg.n_pages // 2, cfg.n_pages))
        main = torch.cuda.current_stream()
        sims = torch.empty(n_hist, dtype=torch.float32, device="cuda")
        pred = torch.empty(1, dtype=torch.int32, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks_gen + 1)]
        torch.cuda.synchronize()
        ev[0].record(main)
        for t in range(n_chunks_gen):
            st.retrieve(q, [None] * cfg.n_pages, (prompts_d[t], prev_d, pc_d, 1), main)
            sel = st.sel_pages.cpu().tolist()  # the host learns the selection
            tiers.request(sel)
            main.wait_event(tiers.ready)
            pk_t, pv_t = tiers.tables()
            st.gather(pk_t, pv_t, main)
            gathered = torch.cuda.Event()
            gathered.record(main)
            if prefetch and t + 1 < n_chunks_gen:
                # predict the next chunk's history chunk (stage 1 on its prompt,
                # on the copy stream) and bring its pages in behind the gather
                with torch.cuda.stream(tiers.stream):
                    ops.hsa_retrieve_chunks(prompts_d[t + 1], prev_d, 1, sims, pred, tiers.stream)
                    nxt = int(pred.cpu())
                tiers.request([j for j in range(cfg.n_pages) if page_chunk[j] == nxt], after=gathered)
            for _ in range(R):
                st.linear(q, e_k, e_v, 0, main)
                st.select(q, tau, True, main)
                st.sparse(q, main)
                st.fuse(x, w_g, main)
            ev[t + 1].record(main)
        torch.cuda.synchronize()
        per = [ev[t].elapsed_time(ev[t + 1]) for t in range(n_chunks_gen)]
        return per, tiers.policy.stats(), tiers.bytes_moved

    run(False)  # warm-up (allocations, first launches)
    od, od_stats, od_bytes = run(False)
    pf, pf_stats, pf_bytes = run(True)
    ms_od, ms_pf = float(np.mean(od[1:])), float(np.mean(pf[1:]))
    print(json.dumps({
        "metric": "ms per generated chunk, pages in tiers", "value": round(ms_pf, 3), "unit": "ms/chunk",
        "n_gpus": 1, "steps": n_chunks_gen, "warmup": 1, "ms_per_step": round(ms_pf, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name + "+tiers", "history_pages": cfg.n_pages, "pages_per_chunk": kp,
                   "device_slots": kp, "host_slots": cfg.n_pages // 2, "stage_repeats": R,
                   "history_chunk_walk": [int(c) for c in targets]},
        "ms_on_demand": round(ms_od, 3), "ms_prefetch": round(ms_pf, 3),
        "exposed_fetch_ms": round(ms_od - ms_pf, 3),
        "per_chunk_ms": {"on_demand": [round(v, 2) for v in od], "prefetch": [round(v, 2) for v in pf]},
        "tier_stats": {"on_demand": od_stats, "prefetch": pf_stats},
        "bytes_moved": {"on_demand": od_bytes, "prefetch": pf_bytes},
    }), flush=True)


def run_single(args, cfg, steps: int, warmup: int, with_cpu: bool, with_peaks: bool = True) -> dict:
    """One layer, one denoising step of a single-step workload: W warm-up
    steps, a per-stage pass of K steps (calls in order on one stream, events
    between them), then K timed steps in the step's own schedule.  Returns
    the benchmark line as a dict."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from synth import Workload
    from sparse_linear_attention_hsa_amd import ops
    from sparse_linear_attention_hsa_amd.ops import make_geom
    from sparse_linear_attention_hsa_amd.step import HsaStep

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = Workload(cfg)
    s = w.small_inputs()
    up = lambda a: torch.from_numpy(a).to(tdt).cuda()
    q, x, e_k, e_v, w_g = (up(s[k]) for k in ("q", "x", "e_k", "e_v", "w_g"))
    k_cur, v_cur = (up(s["k_cur"]), up(s["v_cur"])) if cfg.intra_split else (None, None)
    tau = torch.from_numpy(s["tau"]).cuda()
    keep_host = with_cpu  # the oracle's scoring reads every page
    pk_np, pv_np, pk, pv = [], [], [], []
    with ThreadPoolExecutor(16) as ex:  # pages generated on a thread pool, uploaded in order
        for j, (kj, vj) in enumerate(ex.map(lambda i: (w.page_k(i), w.page_v(i)), range(cfg.n_pages))):
            pk.append(up(kj))
            pv.append(up(vj))
            if keep_host:
                pk_np.append(kj)
                pv_np.append(vj)
            if (j + 1) % 8 == 0 or j + 1 == cfg.n_pages:
                print(f"bench: {cfg.name}: generated {j + 1}/{cfg.n_pages} pages", file=sys.stderr, flush=True)
    geom = make_geom(cfg.n_heads, cfg.head_dim, cfg.frame_h, cfg.frame_w, cfg.frames_per_page,
                     cfg.query_frames, cfg.tile, cfg.n_sel_pages, cfg.rank, cfg.dtype, cfg.intra_split)
    st = HsaStep(geom, cfg.n_pages)
    stream = torch.cuda.current_stream()

    paged = bool(args.paged)
    indexed = bool(args.page_index) or paged
    if indexed:
        st.index_pages(q, pk)  # the page index, built once (outside the timed steps)
        torch.cuda.synchronize()
    prepared = None
    if paged:  # every page laid out once, as when it is written (outside the timed steps)
        prepared = st.prepare_pages(pk, pv)
        torch.cuda.synchronize()
    chunks = None
    if args.chunks:
        from synth import chunk_prompts
        page_chunk, cur, prev, _ = chunk_prompts(cfg, args.pages_per_chunk)
        chunks = (torch.from_numpy(cur).cuda(), torch.from_numpy(prev).cuda(), torch.from_numpy(page_chunk).cuda(),
                  args.chunks)

    def score_stage():
        if chunks is not None:
            st.retrieve(q, [None] * cfg.n_pages if indexed else pk, chunks)
        else:
            st.score(q, pk, use_cache=indexed)

    def one_step():
        # the step's own schedule: the linear branch on a side stream beside
        # block selection and the sparse branch, joined before the fusion
        # (on the current stream, which is the capture stream under --graph)
        if paged:
            st.run_paged(q, prepared, e_k, e_v, w_g, x, tau, k_cur=k_cur, v_cur=v_cur)
        else:
            st.run(q, pk, pv, e_k, e_v, w_g, x, tau, indexed=indexed, chunks=chunks, k_cur=k_cur, v_cur=v_cur)

    def one_step_staged(ev, kev):
        # the same six calls in order on one stream, with events between them
        calls = (score_stage, lambda: st.gather(pk, pv, k_cur=k_cur, v_cur=v_cur),
                 lambda: st.linear(q, e_k, e_v),
                 lambda: st.select(q, tau), lambda: st.sparse(q, kernel_events=kev), lambda: st.fuse(x, w_g))
        if paged:  # the same stages reading the laid-out pages
            tab = {}

            def paged_gather():  # (with intra-chunk keys the chunk is laid out here)
                tab["t"] = st.paged_inputs(prepared, k_cur, v_cur)
                ops.hsa_gather_block_means(geom, tab["t"][2], tab["t"][3], st.kblk_mean)

            calls = (score_stage, paged_gather,
                     lambda: ops.hsa_linear_branch_paged(geom, q, tab["t"][0], tab["t"][1], tab["t"][3], e_k, e_v,
                                                         st.k_proj, st.v_proj, st.o_lin, 0, st.ws),
                     lambda: ops.hsa_block_select(geom, q, None, st.kblk_mean, tau, st.blk_count, st.blk_idx,
                                                  st.blk_mass, st.ws),
                     lambda: ops.hsa_sparse_attn_paged(geom, q, tab["t"][0], tab["t"][1], tab["t"][3], st.blk_count,
                                                       st.blk_idx, st.o_sp, st.ws, kev),
                     lambda: st.fuse(x, w_g))
        for i, fn in enumerate(calls):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # per-stage HIP events over a pass of the same launches issued in order on
    # one stream (events between calls), plus, inside the sparse stage, events
    # around the attention kernel alone (recorded by the library on the same
    # stream).  This pass runs before the timed region, so the timed steps
    # find the GPU in its steady state.
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in STAGES]
           for _ in range(steps)]
    kevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        one_step_staged(evs[k], kevs[k])
    torch.cuda.synchronize()
    # timed region: K whole steps in the step's own schedule (an event after
    # every step gives the per-step spread; events do not synchronise)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    step_ev[0].record(stream)
    for k in range(steps):
        if graph is not None:
            graph.replay()
        else:
            one_step()
        step_ev[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = step_ev[0].elapsed_time(step_ev[-1]) / steps
    per_step = np.array([step_ev[k].elapsed_time(step_ev[k + 1]) for k in range(steps)])
    peaks = measured_peaks() if with_peaks else None

    stage_ms = {name: float(np.mean([evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(steps)]))
                for i, name in enumerate(STAGES)}
    attn_kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in kevs]))

    counts = st.blk_count.cpu().numpy()
    n_sel_total = int(counts.sum())
    scored_pages = cfg.n_pages
    if chunks is not None:  # only the retrieved chunks' pages are read
        pc = chunks[2].cpu().numpy()
        scored_pages = int(np.isin(pc, st.sel_chunks.cpu().numpy()).sum())
    model = stage_model(cfg, n_sel_total, indexed, scored_pages, paged)
    sparse_tf = model["sparse"]["flops"] / (stage_ms["sparse"] * 1e-3) / 1e12
    lin_tf = model["linear"]["flops"] / (stage_ms["linear"] * 1e-3) / 1e12
    peak_tf = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    # Roofline of the dominant kernel: the block-sparse attention kernel
    # (algorithmic flops 4*B*Bk*d per selected (query block, key block) pair,
    # Bk = B without intra-chunk keys; all pairs of the step in one launch)
    # over its own event-timed duration.
    ach = model["sparse"]["flops"] / (attn_kernel_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_tf, "unit": "TFLOP/s",
            "frac": round(ach / peak_tf, 4), "traffic": measured_traffic(cfg.name),
            "kernel": "sparse_attn_kernel", "kernel_ms": round(attn_kernel_ms, 4)}

    out = {
        "metric": METRIC, "value": round(ms, 4), "unit": "ms/chunk", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                   "retrieved_tokens": cfg.history_tokens, "query_tokens": cfg.query_tokens,
                   "history_pages": cfg.n_pages, "block": cfg.block, "rank": cfg.rank,
                   "intra_split": cfg.intra_split, "key_block": cfg.key_block, "active_tokens": cfg.active_tokens,
                   "graph": bool(args.graph), "page_index": indexed, "paged": paged, "chunks": args.chunks,
                   "pages_per_chunk": args.pages_per_chunk if args.chunks else None},
        "ms_per_step_stats": {"median": round(float(np.median(per_step)), 4),
                              "min": round(float(per_step.min()), 4),
                              "p90": round(float(np.percentile(per_step, 90)), 4)},
        "step_tflops": round(sum(m.get("flops", 0) for m in model.values()) / (ms * 1e-3) / 1e12, 1),
        "attended_tflops": round(sparse_tf, 1), "mfma_frac_sparse": round(sparse_tf / peak_tf, 4),
        "peaks_measured": peaks,
        "selected_block_frac": round(n_sel_total / (cfg.n_heads * cfg.n_qblocks * cfg.n_key_blocks), 4),
        "linear_tflops": round(lin_tf, 1),
        "score_gbs": round(model["score"]["bytes"] / (stage_ms["score"] * 1e-3) / 1e9, 1),
        "gather_gbs": round(model["gather"]["bytes"] / (stage_ms["gather"] * 1e-3) / 1e9, 1),
        "hbm_frac_of_8tbs": {k: round(model[k]["bytes"] / (stage_ms[k] * 1e-3) / 8e12, 4) for k in ("score", "gather")},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roof,
    }
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, w, (s, pk_np, pv_np))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c1_full")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="time only the chosen workload (by default c1_full also times c3 and c2 as extra keys)")
    ap.add_argument("--graph", action="store_true", help="replay the step as one HIP graph")
    ap.add_argument("--chunks", type=int, default=0,
                    help="prompt-level retrieval first: keep the K most similar chunks and score only their pages "
                         "(K_p/K pages from each)")
    ap.add_argument("--pages-per-chunk", type=int, default=8, help="history pages per chunk for --chunks")
    ap.add_argument("--tiers", type=int, default=0,
                    help="run this many generated chunks with the pages in tiers, fetched on demand and prefetched")
    ap.add_argument("--tiers-steps", type=int, default=120,
                    help="per-step stages repeated per generated chunk under --tiers (30 layers x 4 steps)")
    ap.add_argument("--page-index", action="store_true",
                    help="score from a page index of mean keys built once before the timed steps "
                         "(as when pages are written) instead of reading every page's keys")
    ap.add_argument("--paged", action="store_true",
                    help="lay the pages out once (as when written) and run the step reading them in place: scoring "
                         "from the page index, no active-buffer copy")
    ap.add_argument("--intra", type=int, default=0,
                    help="intra-chunk keys: the chunk's own tokens follow the retrieved pages in key blocks of "
                         "B/S tokens (S = 2: 48-token blocks beside the 96-token history tiles)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run three device-to-device copies of 1 GiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: this build measures one GPU; --gpus > 1 is not supported "
              "(the HSA step shards by head, see the design notes, but no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    from synth import CONFIGS

    cfg = CONFIGS[args.config]
    if args.paged and (args.chunks or args.tiers or cfg.layers > 1 or cfg.steps > 1):
        print("bench.py: --paged runs the single-step workloads without --chunks / --tiers",
              file=sys.stderr)
        sys.exit(2)
    if args.paged:
        from dataclasses import replace
        cfg = replace(cfg, name=f"{cfg.name}_paged")
    if args.intra:
        from dataclasses import replace
        if args.tiers or args.chunks or cfg.layers > 1 or cfg.steps > 1:
            print("bench.py: --intra runs the single-step workloads without --tiers / --chunks", file=sys.stderr)
            sys.exit(2)
        cfg = replace(cfg, name=f"{cfg.name}_intra{args.intra}", intra_split=args.intra)
        cfg.check()
    if args.tiers:
        return run_tiers(args, cfg)
    if cfg.layers > 1 or cfg.steps > 1:
        return run_stack(args, cfg)
    out = run_single(args, cfg, args.steps, args.warmup, not args.no_cpu_baseline)
    variant = args.graph or args.page_index or args.paged or args.chunks or args.intra
    if args.config == "c1_full" and not variant and not args.no_extra_configs:
        # the head-imbalance and long-history workloads, timed the same way
        # (fewer steps), as extra keys of the same line
        torch.cuda.empty_cache()
        out["extra_configs"] = {}
        for name in ("c3_head_imbalance", "c2_long_history"):
            e = run_single(args, CONFIGS[name], min(args.steps, 20), min(args.warmup, 5), False, with_peaks=False)
            out["extra_configs"][name] = {
                "ms_per_chunk": e["value"], "ms_per_step_stats": e["ms_per_step_stats"],
                "sparse_roofline_frac": e["roofline"]["frac"], "sparse_kernel_ms": e["roofline"]["kernel_ms"],
                "attended_tflops": e["attended_tflops"], "selected_block_frac": e["selected_block_frac"],
                "stages_ms": e["stages_ms"], "history_pages": CONFIGS[name].n_pages}
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
