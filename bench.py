"""Throughput of the ISD step on one MI355X.

A step is one pass of the whole hot path over the batch: isd_attention ->
isd_accept_commit (the accept test, residual resampling and the KV commit of
the accepted rows in one call) (+ isd_lora_delta for the R-ISD workload),
enqueued on one stream.  The MASK-row proposals for the next step (isd_propose, sampling
and argmax policies) are timed in a loop of their own after the steps and
reported under "propose"; they do not enter "value".  Neither do "graph" (the
step replayed from HIP graphs) and "loop" (whole forwards of the multi-step
decoding loop, with its measured tokens per forward).

Inputs are synthetic (workloads/), generated on the host and resident in HBM
before the timed region.  To keep the Infinity Cache (256 MB) from serving
repeated steps, the timed loop rotates over several independent copies of
every input whose total exceeds the cache several times over.  The commit
writes lengths to a second buffer, so every timed step sees the same context
lengths (the committed rows land in slots the next attention does not read).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c32_ctx4k]

Prints one JSON line (see the keys below).  --gpus above 1 is refused: the
step shards by request with no exchange, but this benchmark runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
MALL_BYTES = 256 * 2 ** 20
SAMPLE_FIRST, SAMPLE_EVERY = 5, 10   # timed steps whose calls are bracketed by HIP events


def measured_traffic(cfg_name):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None when there is none for this workload or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_bf16_hbm_traffic_{cfg_name}.md")
    if not os.path.exists(path):
        return None
    want, traffic = None, None
    for line in open(path):
        if line.startswith("kernel_source_sha256:"):
            want = line.split(":", 1)[1].strip()
        elif line.startswith("traffic_bytes_per_launch"):
            traffic = int(line.rsplit(":", 1)[1].strip())
    h = hashlib.sha256()
    for f in ("attention.hip", "device_common.hpp", "isd_internal.hpp"):
        with open(os.path.join(ROOT, "introspective_strided_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return traffic if want == h.hexdigest() else None


def algorithmic_bytes(wl):
    """Bytes each call must move at least once (inputs read once, outputs written once)."""
    cfg = wl.cfg
    s = cfg.elem_bytes
    B, Q, Hq, Hkv, D, N, V = (cfg.batch, cfg.q_rows, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                              cfg.stride_n, cfg.vocab)
    ctx = wl.ctx_lens.astype("int64")
    pages_read = int(((ctx + 15) // 16).sum())
    attn = (int(ctx.sum()) * Hkv * D * 2 * s          # K and V context
            + B * Q * Hq * D * s * 2                     # q in, out
            + B * Q * Hkv * D * s * 2                    # k_new, v_new
            + pages_read * 4 + B * 4)                    # page-table entries, lengths
    accept = (2 * B * (N - 1) * V * s                    # p and q logits, one read
              + B * N * 4 * 2 + B * 4 * 4 + 2 * B * (N - 1) * 4)
    return {"attention": attn, "accept": accept}


def commit_bytes(wl, rows):
    """KV rows committed (read from the stride, written to the pages), plus lengths and counts."""
    cfg = wl.cfg
    return int(round(rows * cfg.n_kv_heads * cfg.head_dim * cfg.elem_bytes * 2 * 2)) + cfg.batch * 12


def lora_bytes(cfg):
    d, r = cfg.lora_dim, cfg.lora_rank
    m = cfg.batch * cfg.stride_n
    return (m * d + d * r + r * d + 2 * m * d) * 2 + m * 4


def lora_report(cfg, ms):
    """isd_lora_delta: time per call, its flops against the bf16 matrix-core peak and its bytes
    against HBM (the rank-128 delta is HBM-bound: about 73 flop per byte)."""
    d, r = cfg.lora_dim, cfg.lora_rank
    m = cfg.batch * cfg.stride_n
    flops = 2 * m * d * r * 2
    by = lora_bytes(cfg)
    return {"what": "isd_lora_delta: rank-128 adapter on the MASK rows of a 4096 -> 4096 projection",
            "gated_rows": m, "avg_call_ms": round(ms, 5), "flops": int(flops), "bytes": int(by),
            "tflops": round(flops / ms / 1e9, 2), "mfma_frac": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "achieved_GBs": round(by / ms / 1e6, 1), "hbm_frac": round(by / ms / 1e6 / HBM_PEAK_GBS, 4)}


def propose_bytes(cfg):
    """MASK-row logits read once, proposals written once."""
    return cfg.batch * cfg.stride_n * (cfg.vocab * cfg.elem_bytes + 4)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = 10.0, max_steps: int = 8):
    """Time the float64 oracle on the host: whole steps (attention for every request, accept,
    commit) of the same workload, repeated until about ``budget_s`` seconds have passed, with
    the BLAS threads pinned to the CPUs this process may run on."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.accept import isd_accept as o_accept
    from oracle.attention import stride_attention
    from oracle.commit import kv_commit as o_commit

    cfg = wl.cfg
    host_cpus = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=host_cpus):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t_start = time.perf_counter()
        steps_done = 0
        accepted = 0
        while steps_done < max_steps:
            stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                             wl.ctx_lens, cfg.page_size)
            res = o_accept(wl.p_logits, wl.q_logits, wl.proposals, wl.req_ids, wl.positions,
                           wl.philox_seed, wl.step + steps_done)
            n_commit = np.array([o.n_commit for o in res])
            o_commit(wl.k_pool, wl.v_pool, wl.page_table, wl.ctx_lens, wl.k_new, wl.v_new, n_commit,
                     cfg.page_size)
            accepted += sum(o.accept_len for o in res)
            steps_done += 1
            if time.perf_counter() - t_start > budget_s:
                break
        elapsed = time.perf_counter() - t_start
    return {
        "value": round(steps_done / elapsed, 4),
        "unit": "verify-steps/s",
        "accepted_tokens_per_s": round(accepted / elapsed, 2),
        "cores": int(threads),
        "host_cpus": host_cpus,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{steps_done} whole steps of the {cfg.name} workload (float64 attention for "
                   f"every request, accept with residual, commit), BLAS threads pinned to the "
                   f"{host_cpus} CPUs of this process"),
        "seconds": round(elapsed, 2),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD published


def r_isd_projections(cfg, dev, stream, reps):
    """The seven projections of one R-ISD layer of the 8B shape (hidden Hq*D, KV Hkv*D, MLP
    3*hidden) at this workload's stride rows, gated (adapter on the MASK rows) and base-only,
    each recorded into a HIP graph and replayed; PyTorch's own linear layers (hipBLASLt) time
    the base projections for comparison."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    from introspective_strided_decoding_amd.r_isd import RIsdProjections, stride_mask_rows

    hidden, kv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    if hidden % 256 or kv % 128:
        return None
    rows = cfg.batch * cfg.q_rows
    proj = RIsdProjections(rows, stride_mask_rows(cfg.batch, cfg.stride_n), hidden=hidden, kv=kv,
                           mlp=3 * hidden, seed=11, device=dev)
    res = {"what": "q, k, v, o, gate, up, down projections of one layer; adapter rank 128 on the MASK rows; "
                   "one isd_gated_linear_group call per set of projections that share an input "
                   "(q/k/v, o, gate/up, down)",
           "rows": rows, "gated_rows": int(proj.mask.numel()), "hidden": hidden, "kv": kv, "mlp": 3 * hidden}

    def replay_ms(gated, mode):
        for _ in range(3):
            proj.run(gated, mode)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            proj.run(gated, mode)
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / reps

    for gated in (True, False):
        ms = replay_ms(gated, "group")
        f, by = proj.flops(gated), proj.bytes(gated)
        res["gated" if gated else "base"] = {
            "ms": round(ms, 5), "tflops": round(f / ms / 1e9, 1),
            "mfma_frac": round(f / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "GBs": round(by / ms / 1e6, 1), "hbm_frac": round(by / ms / 1e6 / HBM_PEAK_GBS, 4),
            "flops": int(f), "bytes": int(by)}
    # one isd_gated_linear call per projection, siblings on two streams
    per = {"gated_ms": round(replay_ms(True, "overlap"), 5), "base_ms": round(replay_ms(False, "overlap"), 5)}
    per["alpha"] = round(per["gated_ms"] / per["base_ms"], 4)
    res["per_projection_calls"] = per
    res["alpha"] = round(res["gated"]["ms"] / res["base"]["ms"], 4)
    t_mfma = proj.flops(False) / (MFMA_BF16_PEAK_TFLOPS * 1e9)
    t_hbm = proj.bytes(False) / (HBM_PEAK_GBS * 1e6)
    res["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
    res["base_frac_of_bound"] = round(max(t_mfma, t_hbm) / res["base"]["ms"], 4)
    # the same base projections through torch.nn.functional.linear, one stream: one call per
    # projection, and one call per group on the group's weights concatenated (as a fused
    # q/k/v or gate/up layer stores them)
    def torch_ms(pairs):
        for _ in range(3):
            for x, w in pairs:
                F.linear(x, w)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            for x, w in pairs:
                F.linear(x, w)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    from introspective_strided_decoding_amd.r_isd import GROUPS
    pairs = [(t["X"], t["W_t"]) for t in proj.p.values()]
    res["torch_linear_base_ms"] = round(torch_ms(pairs), 5)
    pairs = [(proj.p[grp[0]]["X"], torch.cat([proj.p[nm]["W_t"] for nm in grp])) for grp in GROUPS]
    res["torch_linear_fused_base_ms"] = round(torch_ms(pairs), 5)
    del proj, pairs
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="c32_ctx4k")
    ap.add_argument("--sets", type=int, default=0, help="input copies rotated in the timed loop (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-loop", action="store_true", help="skip the decoding-loop measurement")
    ap.add_argument("--no-r-isd", action="store_true", help="skip the R-ISD layer projections")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device copy before the timed loop (a known-size reference "
                         "for hardware traffic counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the ISD step shards by request with no exchange, "
              "and this build measures the single-GPU step (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from introspective_strided_decoding_amd.step import DeviceStep
    from workloads import get_config, make_workload

    cfg = get_config(args.config)
    t_gen = time.perf_counter()
    loop_forwards = 0 if args.no_loop else max(20, min(200, args.steps))
    wl = make_workload(cfg, with_mask_logits=True)
    t_gen = time.perf_counter() - t_gen
    nbytes = algorithmic_bytes(wl)
    step_bytes = nbytes["attention"] + nbytes["accept"]
    per_set = step_bytes + (lora_bytes(cfg) if cfg.lora else 0) + propose_bytes(cfg)
    sets = args.sets or max(2, min(8, int(np.ceil(4 * MALL_BYTES / per_set))))

    torch.cuda.set_device(0)
    dev = "cuda:0"
    base = DeviceStep.from_arrays(wl, device=dev, max_ctx=int(wl.ctx_lens.max()))
    steps = [base]
    for _ in range(sets - 1):
        st = DeviceStep.from_arrays(wl, device=dev, max_ctx=int(wl.ctx_lens.max()))
        steps.append(st)
    use_lora = cfg.lora
    if use_lora:
        try:
            base.lora_delta()
            torch.cuda.synchronize()
        except Exception as e:  # LoRA entry point missing in this build
            print(f"bench: LoRA delta not run ({e})", file=sys.stderr)
            use_lora = False

    stream = torch.cuda.current_stream()

    def one_step(st, step, ev=None):
        """One verify step; ``ev``: events around its calls (attention, accept + commit, LoRA)."""
        if ev is not None:
            ev[0].record(stream)
        st.attention()
        if ev is not None:
            ev[1].record(stream)
        st.accept_commit(step=step)
        if ev is not None:
            ev[2].record(stream)
        if use_lora:
            st.lora_delta()
            if ev is not None:
                ev[3].record(stream)

    if args.calibrate_copy:
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        one_step(steps[i % sets], wl.step + i)
    torch.cuda.synchronize()

    # Every timed step draws with its own Philox step.  HIP events bracket the calls of
    # every EVERY-th step only (an event costs the stream about 2 us), so the per-kernel
    # figures are measured live in the timed region while the step rate is not skewed.
    sampled = {i for i in range(SAMPLE_FIRST, args.steps, SAMPLE_EVERY)} or {0}
    events = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for i in sampled}
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t_base = wl.step + args.warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span[0].record(stream)
    for i in range(args.steps):
        one_step(steps[i % sets], t_base + i, events.get(i))
    span[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    attn_each = np.array([e[0].elapsed_time(e[1]) for e in events.values()])
    accept_each = np.array([e[1].elapsed_time(e[2]) for e in events.values()])
    lora_each = np.array([e[2].elapsed_time(e[3]) for e in events.values()]) if use_lora else None
    attn_ms = float(np.mean(attn_each))
    accept_ms = float(np.mean(accept_each))
    pct = lambda x: {"p10": round(float(np.percentile(x, 10)), 5), "p50": round(float(np.percentile(x, 50)), 5),
                     "p90": round(float(np.percentile(x, 90)), 5)}
    ms_per_step = elapsed * 1e3 / args.steps
    steps_per_s = args.steps / elapsed
    gpu_ms_per_step = span[0].elapsed_time(span[1]) / args.steps

    # the timed steps' draws again, untimed: accepted / committed tokens and committed rows
    # averaged over every timed step (inputs are unchanged between steps, so step i draws
    # exactly what it drew in the timed loop)
    acc_tot, out_tot, cm_tot = (torch.zeros((), dtype=torch.int64, device=dev) for _ in range(3))
    for i in range(args.steps):
        st = steps[i % sets]
        st.accept(step=t_base + i)
        acc_tot += st.accept_len.sum()
        out_tot += st.n_out.sum()
        cm_tot += st.n_commit.sum()
    accepted_per_step = float(acc_tot.item()) / args.steps
    committed_per_step = float(out_tot.item()) / args.steps
    committed_rows_per_step = float(cm_tot.item()) / args.steps

    # the same steps replayed from HIP graphs (one recorded step per input set)
    graph = None
    if not args.no_graph:
        graphs = [st.capture() if not use_lora else None for st in steps]
        if all(g is not None for g in graphs):
            # the recorded step also draws the next proposals; time it against eager steps that do too
            for i in range(args.warmup):
                graphs[i % sets].replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % sets].replay()
            torch.cuda.synchronize()
            g_elapsed = time.perf_counter() - t0
            for i in range(args.warmup):
                steps[i % sets].run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                steps[i % sets].run()
            torch.cuda.synchronize()
            e_elapsed = time.perf_counter() - t0
            graph = {"what": "attention, accept, commit and sampled proposals per step",
                     "graph_steps_per_s": round(args.steps / g_elapsed, 2),
                     "eager_steps_per_s": round(args.steps / e_elapsed, 2),
                     "graph_ms_per_step": round(g_elapsed * 1e3 / args.steps, 5)}
            del graphs
            # the verify step alone (what "value" times eagerly), recorded and replayed
            vgraphs = []
            for st in steps:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    one_step(st, wl.step)
                vgraphs.append(g)
            for i in range(args.warmup):
                vgraphs[i % sets].replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                vgraphs[i % sets].replay()
            torch.cuda.synchronize()
            v_elapsed = time.perf_counter() - t0
            graph["verify_step_graph_steps_per_s"] = round(args.steps / v_elapsed, 2)
            graph["verify_step_graph_ms_per_step"] = round(v_elapsed * 1e3 / args.steps, 5)
            del vgraphs

    # the decoding loop: whole forwards (attention, accept, proposals, bookkeeping, commit in place)
    loop = None
    if loop_forwards and not use_lora:
        # every forward verifies proposals drawn from the q rows it is tested against, so the
        # per-position acceptance is the workload's target
        # the same workload with page room for the tokens the loop commits
        room = 2 * loop_forwards + 16          # the eager forwards, then the same number replayed
        lwl = make_workload(cfg, with_mask_logits=True, extra_tokens=room * cfg.stride_n)
        lp = DeviceStep.from_arrays(lwl, device=dev, max_ctx=int(lwl.ctx_lens.max()) + room * cfg.stride_n,
                                    commit_in_place=True)
        del lwl
        row0 = lp.mask_logits[:, :1].clone()
        lp.mask_logits.copy_(torch.cat([row0, lp.q_logits], dim=1))
        lp.loop_start()
        for t in range(4):
            lp.loop_forward(step=t)
        torch.cuda.synchronize()
        tok0 = int(lp.extra["tokens"].sum().item())
        fw0 = int(lp.extra["forwards"].sum().item())
        t0 = time.perf_counter()
        for t in range(4, 4 + loop_forwards):
            lp.loop_forward(step=t)
        torch.cuda.synchronize()
        l_elapsed = time.perf_counter() - t0
        tokens = int(lp.extra["tokens"].sum().item()) - tok0
        fws = int(lp.extra["forwards"].sum().item()) - fw0
        loop = {"what": "decoding loop: attention, accept, sampled proposals, bookkeeping, commit in place",
                "forwards": loop_forwards,
                "forwards_per_s": round(loop_forwards / l_elapsed, 2),
                "tokens_per_s": round(tokens / l_elapsed, 1),
                "tpf": round(tokens / fws, 4),
                "ms_per_forward": round(l_elapsed * 1e3 / loop_forwards, 5)}
        # the same loop with one forward recorded into a HIP graph and replayed (Philox steps
        # from the device forward counts)
        for _ in range(4):
            lp.loop_forward(device_step=True)
        torch.cuda.synchronize()
        lgraph = lp.capture_loop_forward()
        tok0 = int(lp.extra["tokens"].sum().item())
        fw0 = int(lp.extra["forwards"].sum().item())
        t0 = time.perf_counter()
        for _ in range(loop_forwards):
            lgraph.replay()
        torch.cuda.synchronize()
        g_elapsed = time.perf_counter() - t0
        tokens = int(lp.extra["tokens"].sum().item()) - tok0
        fws = int(lp.extra["forwards"].sum().item()) - fw0
        loop["graph"] = {"forwards_per_s": round(loop_forwards / g_elapsed, 2),
                         "tokens_per_s": round(tokens / g_elapsed, 1), "tpf": round(tokens / fws, 4),
                         "ms_per_forward": round(g_elapsed * 1e3 / loop_forwards, 5)}
        del lgraph
        del lp

    # MASK-row proposals, timed on their own (both policies)
    from introspective_strided_decoding_amd._lib import PROPOSE_ARGMAX, PROPOSE_SAMPLE
    prop = {}
    pbytes = propose_bytes(cfg)
    for name, mode in (("sample", PROPOSE_SAMPLE), ("argmax", PROPOSE_ARGMAX)):
        for i in range(min(args.warmup, 10)):
            steps[i % sets].propose(mode=mode)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(20, args.steps // 3))]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(pev):
            a.record(stream)
            steps[i % sets].propose(mode=mode)
            b.record(stream)
        torch.cuda.synchronize()
        pms = float(np.mean([a.elapsed_time(b) for a, b in pev]))
        prop[name] = {"avg_call_ms": round(pms, 5), "achieved_GBs": round(pbytes / pms / 1e6, 1),
                      "frac": round(pbytes / pms / 1e6 / HBM_PEAK_GBS, 4)}
    prop["bytes_per_call"] = int(pbytes)
    prop["steps_per_s_with_sampled_proposals"] = round(1e3 / (ms_per_step + prop["sample"]["avg_call_ms"]), 2)

    r_isd = None if args.no_r_isd else r_isd_projections(cfg, dev, stream, reps=max(20, args.steps // 3))
    if r_isd is not None:
        # one layer's attention (this step's launch) plus its seven projections, gated over
        # base-only: the adapter's share once attention is in the layer (norms, rotary
        # embedding, the SiLU product and residual adds left out)
        r_isd["attention_ms"] = round(attn_ms, 5)
        r_isd["alpha_with_attention"] = round((attn_ms + r_isd["gated"]["ms"]) / (attn_ms + r_isd["base"]["ms"]), 4)

    c_bytes = commit_bytes(wl, committed_rows_per_step)
    total_bytes = step_bytes + c_bytes + (lora_bytes(cfg) if use_lora else 0)
    accept_bytes = nbytes["accept"] + c_bytes

    out = {
        "metric": "ISD verify-steps/s + accepted tokens/s at concurrency 32, N=4; % HBM peak",
        "value": round(steps_per_s, 2),
        "unit": "verify-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "ctx": cfg.ctx or list(cfg.ctx_range),
                   "stride_n": cfg.stride_n, "q_rows": cfg.q_rows, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "vocab": cfg.vocab,
                   "page_size": cfg.page_size, "lora": bool(use_lora), "input_sets": sets,
                   "description": cfg.description},
        "accepted_tokens_per_s": round(accepted_per_step * steps_per_s, 1),
        "committed_tokens_per_s": round(committed_per_step * steps_per_s, 1),
        "request_steps_per_s": round(cfg.batch * steps_per_s, 1),
        "accepted_per_step": round(accepted_per_step, 3),
        "committed_per_step": round(committed_per_step, 3),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "event_ms": {"samples": len(events), "attention": pct(attn_each), "accept_commit": pct(accept_each)},
        "step_hbm": {"bytes": int(total_bytes), "achieved_GBs": round(total_bytes / ms_per_step / 1e6, 1),
                     "frac": round(total_bytes / ms_per_step / 1e6 / HBM_PEAK_GBS, 4)},
        "roofline": {
            "kernel": "attn_bf16 (isd_attention: paged stride attention, one launch)",
            "bound": "hbm",
            "achieved": round(nbytes["attention"] / attn_ms / 1e6, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes["attention"] / attn_ms / 1e6 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name),
            "bytes_per_launch": int(nbytes["attention"]),
            "avg_launch_ms": round(attn_ms, 5),
        },
        "accept": {
            "what": "isd_accept_commit: row normalisers, accept decision (its own launch, or inside "
                    "every residual pass workgroup on small batches), residual pass, residual selection "
                    "with the KV commit",
            "bound": "hbm",
            "bytes_per_call": int(accept_bytes),
            "avg_call_ms": round(accept_ms, 5),
            "achieved_GBs": round(accept_bytes / accept_ms / 1e6, 1),
            "frac": round(accept_bytes / accept_ms / 1e6 / HBM_PEAK_GBS, 4),
        },
        "lora": None if lora_each is None else lora_report(cfg, float(np.mean(lora_each))),
        "propose": prop,
        "graph": graph,
        "loop": loop,
        "r_isd": r_isd,
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
