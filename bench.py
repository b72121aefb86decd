"""Benchmark of one SpecOPD branch-scoring step on one MI355X.

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM: tree-masked attention of every branch node against the trunk
cache (specopd_tree_attn_fwd), then the E2E-TV surrogate forward and gradient
over the scored rows (specopd_e2etv_fwd_bwd).  The timed steps replay the step
captured once as a HIP graph (every kernel of both calls runs in every
replay); --eager times plain calls, and the JSON line carries both.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

Prints one JSON line.  `value` is scored branch rows per second through the
whole step.  `roofline` describes the kernel that takes most of the step,
timed with HIP events on the stream it runs on; `roofline_attn` /
`roofline_loss` give both parts.  `prefill` measures, separately, the trunk
prefill that fills the cache (specopd_prefill_fwd) on the workload's trunks.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload (reported, not a target).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "branch scoring rows/s (tree attn, MFMA util) + E2E-TV rows/s (HBM GB/s)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector


def attn_flops(cfg, anchors):
    """Algorithmic attention FLOPs: QK^T and PV over unmasked keys only,
    4*D*Hq per (row, visible key); node j sees a_b + 1 trunk keys and
    depth(j) + 1 branch keys."""
    import numpy as np
    depth = np.asarray(cfg.depth, np.float64)
    a = anchors.astype(np.float64)                       # [T][B]
    keys = (a[:, :, None] + 2.0 + depth[None, None, :]).sum()
    return 4.0 * cfg.D * cfg.Hq * keys


def loss_bytes(cfg, grad_bytes=4):
    """Algorithmic E2E-TV bytes: read draft and target once, write the
    gradient once, plus 12 bytes of per-row scalars."""
    s_in = 2 if cfg.dtype == "bf16" else 4
    return cfg.N * cfg.V * (2 * s_in + grad_bytes) + 12 * cfg.N


def measured_traffic(kernel_tag, src_files):
    """HBM bytes per launch of a kernel from the committed counter summary
    (profiles/<kernel_tag>.txt), or None when the kernel source has changed
    since the counters were taken (the summary records its sha256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", kernel_tag + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in src_files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if kv.get("source_sha256") != h.hexdigest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_graph(step, stream, steps):
    """ms per step over `steps` replays of step() captured as one HIP graph
    (warmed up on a side stream first, one untimed replay)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(None)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(None)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / steps


def prefill_flops(cfg):
    """Algorithmic FLOPs of one trunk's causal prefill: token s reads s + 1
    keys, 4*D*Hq per (row, key)."""
    return 4.0 * cfg.D * cfg.Hq * cfg.L * (cfg.L + 1) / 2.0


def bench_prefill(sd, wl, seed, steps, warmup, dev, stream):
    """Trunk prefill of the workload's trunks (specopd_prefill_fwd), timed on
    its own: it precedes the scoring step and is not part of it."""
    import torch
    from synthetic import gen_prefill
    ac = wl.attn
    pi = gen_prefill(ac, seed, device=dev, cid=wl.cid)
    desc = sd.prefill_desc(ac.T, ac.L, ac.Hq, ac.Hkv, ac.D, pi["q"].dtype)
    ws = sd.workspace(sd.specopd_prefill_workspace_size(desc), dev)
    out, ck, cv = torch.empty_like(pi["q"]), torch.empty_like(pi["k"]), torch.empty_like(pi["v"])

    def call():
        sd.specopd_prefill_fwd(desc, pi["q"], pi["k"], pi["v"], ck, cv, out, ws)

    for _ in range(max(1, warmup)):
        call()
    n = max(1, min(steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / n
    sd.specopd_kernel_timing(True)
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    tot, cnt = sd.specopd_kernel_time(2)
    sd.specopd_kernel_timing(False)
    kern_ms = tot / cnt  # one launch per trunk
    fl = prefill_flops(ac)
    tf = fl / (kern_ms / 1e3) / 1e12
    peak = BF16_PEAK_TFLOPS if ac.dtype == "bf16" else FP32_PEAK_TFLOPS
    t_pf = measured_traffic(f"prefill_mfma_{wl.name}",
                            ["speculative_decoding_drafter_amd/csrc/tree_attn_mfma.hip",
                             "speculative_decoding_drafter_amd/csrc/device_common.h",
                             "speculative_decoding_drafter_amd/csrc/internal.h",
                             "speculative_decoding_drafter_amd/build.py"])
    return {
        "metric": "trunk prefill tokens/s", "value": ac.T * ac.L / (call_ms / 1e3),
        "unit": "tokens/s", "calls": n, "call_ms": call_ms,
        "config": {"T": ac.T, "L": ac.L, "Hq": ac.Hq, "Hkv": ac.Hkv, "D": ac.D, "dtype": ac.dtype},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": tf / peak,
                     "traffic": None if t_pf is None else t_pf / (kern_ms / 1e3) / 1e9,
                     "traffic_unit": "GB/s", "traffic_bytes_per_launch": t_pf,
                     "kernel": "tree_attn_mfma_kernel<D, true> (specopd_prefill_fwd, one launch per trunk)",
                     "ms": kern_ms, "alg_flops_per_launch": fl},
    }


def cpu_baseline(wl, attn_inp_cpu, loss_inp_cpu, budget_s=12.0):
    """The fp64 oracle as it stands, single BLAS thread, on a bounded sample:
    whole branches (every node, every head) of attention and their loss rows,
    in a seeded order, going round the branches again until budget_s of CPU
    work.  Returns scored rows per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    rows = 0
    t_total = 0.0
    nb = 0
    with threadpool_limits(limits=1):
        cfg = wl.attn if wl.attn is not None else None
        lc = wl.loss
        R = lc.R
        order = np.random.default_rng(0).permutation(R)
        for i in range(1 << 30):
            r = order[i % R]
            t0 = time.perf_counter()
            if cfg is not None:
                t, b = divmod(int(r), cfg.B)
                if t < cfg.T:
                    c = attn_inp_cpu
                    oracle.tree_attention(c["trunk_k"], c["trunk_v"], c["q"], c["k"], c["v"],
                                          c["anchors"], c["parent"], c["pos"], branches=[(t, b)])
            d = loss_inp_cpu
            oracle.e2etv_branch(d["draft"][r], d["target"][r], d["parent"][r].numpy(), float(lc.N))
            t_total += time.perf_counter() - t0
            rows += lc.Wn
            nb += 1
            if t_total >= budget_s:
                break
    return rows / t_total, nb, t_total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (default: the 8B-shaped layer)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the trunk-prefill measurement")
    ap.add_argument("--eager", action="store_true",
                    help="time plain calls instead of replays of the step captured as a HIP graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the scoring path runs on one GPU; --gpus {args.gpus} is not supported "
              "(trunks, and whole branches of the loss, would be the units sharded across GPUs; "
              "only the loss numerators would then be summed across them).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_drafter_amd as sd
    from synthetic import WORKLOADS, gen_attn, gen_loss

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    wl = WORKLOADS[args.workload]
    torch.manual_seed(args.seed)

    ai = gen_attn(wl.attn, args.seed, device=dev, cid=wl.cid) if wl.attn is not None else None
    li = gen_loss(wl.loss, args.seed, device=dev, cid=wl.cid)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    if ai is not None:
        ac = wl.attn
        adesc = sd.tree_attn_desc(ac.T, ac.L, ac.B, ac.Wn, ac.Hq, ac.Hkv, ac.D, ai["q"].dtype)
        aws = sd.workspace(sd.specopd_tree_attn_workspace_size(adesc), dev)
        aout = torch.empty_like(ai["q"])
    lc = wl.loss
    ldesc = sd.e2etv_desc(lc.R, lc.Wn, lc.V, li["draft"].dtype, torch.float32)
    lws = sd.workspace(sd.specopd_e2etv_workspace_size(ldesc), dev)
    alpha = torch.empty((lc.R, lc.Wn), dtype=torch.float32, device=dev)
    prefix = torch.empty_like(alpha)
    loss = torch.empty(3, dtype=torch.float64, device=dev)
    grad = torch.empty((lc.R, lc.Wn, lc.V), dtype=torch.float32, device=dev)

    def attn_call():
        sd.specopd_tree_attn_fwd(adesc, ai["trunk_k"], ai["trunk_v"], ai["q"], ai["k"], ai["v"],
                                 ai["anchors"], ai["parent"], ai["pos"], aout, aws)

    def loss_call():
        sd.specopd_e2etv_fwd_bwd(ldesc, li["draft"], li["target"], li["parent"], alpha, prefix,
                                 loss, grad, lws)

    def step(ev=None):
        if ai is not None:
            if ev is not None:
                ev[0].record(stream)
            attn_call()
            if ev is not None:
                ev[1].record(stream)
        loss_call()
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy > 0:
        # a plain copy of known size: hardware byte counters are read for it
        # too, and the ratio converts the loss kernel's counters to bytes
        nbytes = args.calibrate_copy << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    # the same steps again with the library recording HIP events around each
    # call's main kernel, so the rooflines divide by the kernel's own duration
    # (a separate pass: the extra event records would otherwise add to the
    # timed steps)
    sd.specopd_kernel_timing(True)
    for i in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    kern_ms = {}
    for which in (0, 1):
        tot, cnt = sd.specopd_kernel_time(which)
        kern_ms[which] = tot / cnt if cnt else None
    sd.specopd_kernel_timing(False)
    # a timed run only counts if every branch came out well formed
    if ai is not None and sd.specopd_tree_attn_device_status(adesc, aws) != 0:
        raise SystemExit("tree attention reported malformed branches")
    if sd.specopd_e2etv_device_status(ldesc, lws) != 0:
        raise SystemExit("E2E-TV reported malformed or timed-out branches")
    eager_ms_step = t_start.elapsed_time(t_end) / args.steps
    # The timed steps: the whole step (every kernel of both calls) captured
    # once as a HIP graph and replayed, which removes the host launch gaps
    # between its kernels; --eager times the plain calls instead (above, with
    # per-call events).
    graph_ms_step = None
    graph_note = None
    if not args.eager:
        try:
            graph_ms_step = time_graph(step, stream, args.steps)
        except RuntimeError as exc:  # capture refused: the eager timing stands
            torch.cuda.synchronize()
            graph_note = f"graph capture failed ({exc}); eager calls timed"
    ms_step = graph_ms_step if graph_ms_step is not None else eager_ms_step
    attn_call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) if ai is not None else 0.0
    loss_call_ms = float(np.mean([(e[1] if ai is not None else e[0]).elapsed_time(e[2]) for e in evs])) \
        if ai is not None else float(np.mean([t_start.elapsed_time(t_end) / args.steps]))
    attn_ms = kern_ms[0] if kern_ms[0] else attn_call_ms
    loss_ms = kern_ms[1] if kern_ms[1] else loss_call_ms

    N = lc.N
    rows_per_s = N / (ms_step / 1e3)
    res = {
        "metric": METRIC, "value": rows_per_s, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if lc.dtype == "bf16" else "f32", "data": "synthetic",
        "graph": graph_ms_step is not None, "eager_ms_per_step": eager_ms_step,
    }
    if graph_note:
        res["graph_note"] = graph_note
    conf = {"workload": f"{wl.name} (workload {wl.cid})", "scored_rows": N,
            "loss": {"R": lc.R, "Wn": lc.Wn, "V": lc.V, "logits": lc.dtype, "grad": "f32"}}
    lb = loss_bytes(lc)
    loss_gbs = lb / (loss_ms / 1e3) / 1e9
    t_loss = measured_traffic(f"e2etv_resident_{wl.name}",
                              ["speculative_decoding_drafter_amd/csrc/e2etv.hip",
                               "speculative_decoding_drafter_amd/csrc/device_common.h",
                               "speculative_decoding_drafter_amd/csrc/internal.h",
                               "speculative_decoding_drafter_amd/build.py"])
    roof_loss = {"bound": "hbm", "achieved": loss_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": loss_gbs / HBM_PEAK_GBS,
                 "traffic": None if t_loss is None else t_loss / (loss_ms / 1e3) / 1e9,
                 "traffic_bytes_per_launch": t_loss,
                 "kernel": "e2etv_resident_kernel (specopd_e2etv_fwd_bwd)", "ms": loss_ms,
                 "call_ms": loss_call_ms,
                 "alg_bytes_per_launch": lb}
    roofs = {"loss": roof_loss}
    if ai is not None:
        ac = wl.attn
        conf["attn"] = {"T": ac.T, "L": ac.L, "B": ac.B, "Wn": ac.Wn, "Hq": ac.Hq, "Hkv": ac.Hkv,
                        "D": ac.D, "dtype": ac.dtype}
        fl = attn_flops(ac, ai["anchors"].cpu().numpy())
        tf = fl / (attn_ms / 1e3) / 1e12
        peak = BF16_PEAK_TFLOPS if ac.dtype == "bf16" else FP32_PEAK_TFLOPS
        t_attn = measured_traffic(f"tree_attn_mfma_{wl.name}",
                                  ["speculative_decoding_drafter_amd/csrc/tree_attn_mfma.hip",
                                   "speculative_decoding_drafter_amd/csrc/device_common.h",
                               "speculative_decoding_drafter_amd/csrc/internal.h",
                               "speculative_decoding_drafter_amd/build.py"])
        roofs["attn"] = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                         "frac": tf / peak,
                         "traffic": None if t_attn is None else t_attn / (attn_ms / 1e3) / 1e9,
                         "traffic_unit": "GB/s", "traffic_bytes_per_launch": t_attn,
                         "kernel": "tree_attn_mfma_kernel (specopd_tree_attn_fwd)",
                         "ms": attn_ms, "call_ms": attn_call_ms, "alg_flops_per_launch": fl}
        res["attn_rows_per_s"] = ac.rows / (attn_call_ms / 1e3)
    res["loss_rows_per_s"] = N / (loss_call_ms / 1e3)
    res["config"] = conf
    dom = max(roofs, key=lambda k: roofs[k]["ms"])
    res["roofline"] = roofs[dom]
    res["roofline_loss"] = roofs["loss"]
    if "attn" in roofs:
        res["roofline_attn"] = roofs["attn"]

    if ai is not None and not args.no_prefill:
        res["prefill"] = bench_prefill(sd, wl, args.seed, args.steps, args.warmup, dev, stream)

    if not args.no_cpu:
        ai_c = {k: v.cpu() for k, v in ai.items()} if ai is not None else None
        li_c = {k: v.cpu() for k, v in li.items()}
        v_cpu, nb, secs = cpu_baseline(wl, ai_c, li_c, args.cpu_budget)
        res["cpu_baseline"] = {
            "value": v_cpu, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{nb} whole branches of {lc.R}, seeded order, repeating ({nb * lc.Wn} scored "
                      f"rows: tree attention over all heads + E2E-TV fwd/grad), fp64 numpy, "
                      f"1 BLAS thread, {secs:.1f} s",
        }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
