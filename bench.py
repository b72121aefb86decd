"""Benchmark of one SpecOPD branch-scoring step on one MI355X.

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM: tree-masked attention of every branch node against the trunk
cache (specopd_tree_attn_fwd), then the E2E-TV surrogate forward and gradient
over the scored rows (specopd_e2etv_fwd_bwd).  The timed steps replay the step
captured once as a HIP graph (every kernel of both calls runs in every
replay); --eager times plain calls, and the JSON line carries both.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--also 2,5]

Prints one JSON line for the workload (default: the batch of 8 trunks of
8192 tokens, 128 branches of 16 nodes each, 32/8 heads of 128, and its
16,384 x 151,936 bf16 logit rows -- the largest configuration on one GPU).
`value` is scored branch rows per second through the whole step.  `roofline`
describes the kernel that takes most of the step, timed with HIP events on
the stream it runs on; `roofline_attn` / `roofline_loss` give both parts,
with the HBM bytes and matrix-core / vector-ALU busy fractions of the
rocprofv3 counter summaries under profiles/ while those match the kernel
sources.  `other_workloads` repeats the measurement for the --also
workloads.  `prefill` measures, separately, the trunk prefill that fills the
cache (specopd_prefill_fwd) on the workload's trunks, and `gdn` the branch
scoring of a linear-attention (GDN) target by indexed state replay
(specopd_gdn_replay_fwd) on the workload's trunks and tree, and `qsa` the block
selection of a sparse-attention (QSA) target with branch-consistent indexer
groups (specopd_qsa_select_fwd), and `lmhead` the E2E-TV loss computed from
the two models' LM heads without storing logits (specopd_lmhead_e2etv_fwd_bwd,
on the 8B-layer shape).  `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same workload, on one core and
on every usable core (reported, not a target).
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


FP32_FMA_TFLOPS = 78.6         # the fp32 vector rate without packed-FP32 instructions


def gdn_flops(cfg, anchors):
    """Algorithmic FLOPs of a GDN replay call: per head, every replayed trunk
    token and every branch node is one gated delta-rule update (S k and the
    rank-1 update, 4 D^2), every node one read (S q, 2 D^2); a branch
    replays the (a + 1) mod C trunk tokens after its checkpoint once."""
    import numpy as np
    rep = float(((anchors.astype(np.int64) + 1) % cfg.C).sum())
    nodes = float(cfg.T * cfg.B * cfg.Wn)
    D2 = float(cfg.D) * cfg.D
    return cfg.H * (4.0 * D2 * (rep + nodes) + 2.0 * D2 * nodes)


def bench_gdn(sd, wl, seed, steps, warmup, dev, stream):
    """GDN branch replay (specopd_gdn_replay_fwd) for a linear-attention
    target on the workload's trunks and tree, timed on its own: it is the
    scoring step's counterpart for GDN layers, not part of the GQA step."""
    import torch
    from synthetic import gen_gdn
    gc = wl.gdn
    gi = gen_gdn(gc, seed, device=dev, cid=wl.cid)
    out, desc, ws = sd.gdn_replay(gi, C=gc.C)

    def call():
        sd.gdn_replay(gi, C=gc.C, ws=ws, out=out)

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
    tot, cnt = sd.specopd_kernel_time(3)
    sd.specopd_kernel_timing(False)
    if sd.specopd_gdn_device_status(desc, ws) != 0:
        raise SystemExit("GDN replay reported malformed branches")
    kern_ms = tot / cnt
    fl = gdn_flops(gc, gi["anchors"].cpu().numpy())
    tf = fl / (kern_ms / 1e3) / 1e12
    rows = gc.T * gc.B * gc.Wn
    pg = profile_summary(f"gdn_replay_{wl.name}", GDN_SRC)
    t_g = _counter(pg, "hbm_bytes_per_launch")
    res = {
        "metric": "GDN branch rows/s (indexed state replay)", "value": rows / (call_ms / 1e3),
        "unit": "rows/s", "calls": n, "call_ms": call_ms,
        "config": {"T": gc.T, "L": gc.L, "B": gc.B, "Wn": gc.Wn, "H": gc.H, "D": gc.D, "C": gc.C,
                   "dtype": gc.dtype},
        "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / FP32_PEAK_TFLOPS, "peak_without_packed_fp32": FP32_FMA_TFLOPS,
                     "frac_without_packed_fp32": tf / FP32_FMA_TFLOPS,
                     "traffic": None if t_g is None else t_g / (kern_ms / 1e3) / 1e9,
                     "traffic_unit": "GB/s", "traffic_bytes_per_launch": t_g,
                     "valu_busy_pct": _counter(pg, "valu_busy_pct"),
                     "kernel": "gdn_replay_kernel (specopd_gdn_replay_fwd)", "ms": kern_ms,
                     "alg_flops_per_launch": fl},
    }
    del gi, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


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
    t_pf = _counter(profile_summary(f"prefill_mfma_{wl.name}", ATTN_SRC), "hbm_bytes_per_launch")
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


_CPU = {}


def _cpu_init():
    from threadpoolctl import threadpool_limits
    import torch
    torch.set_num_threads(1)
    _CPU["lim"] = threadpool_limits(limits=1)


def _cpu_branch(i):
    """One whole branch of the sample through the oracle: tree attention of
    every node and head, then its E2E-TV rows (forward and gradient)."""
    import oracle
    d = _CPU
    b = i % d["nb"]
    if d["attn"] is not None:
        tk, tv, q, k, v, anc, par, pos = d["attn"]
        oracle.tree_attention_branch(tk, tv, q[b], k[b], v[b], anc[b], par[b], pos[b])
    oracle.e2etv_branch(d["draft"][b], d["target"][b], d["lparent"][b], d["count"])
    return b


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, seed, budget_s=16.0, max_workers=16):
    """The fp64 oracle as it stands on a bounded sample of the workload: whole
    branches (tree attention of every node and head against the full trunk,
    then the branch's E2E-TV rows with the workload's global count), drawn
    from the same configuration on the host.  Runs before anything touches
    the GPU, in forked worker processes, each with one BLAS thread: first one
    worker for about budget_s/2, then every usable core (at most max_workers)
    for about as long.  Returns (rows/s on all cores, rows/s on one core,
    workers, branches timed, seconds)."""
    import multiprocessing as mp
    import numpy as np
    from synthetic import gen_attn, gen_loss, shrink_attn, shrink_loss
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    nb = min(wl.loss.R, 2 * workers)
    lc = wl.loss
    li = gen_loss(shrink_loss(lc, R=nb), seed, device="cpu", cid=wl.cid)
    _CPU.update(nb=nb, draft=li["draft"], target=li["target"], lparent=li["parent"].numpy(),
                count=float(lc.N), attn=None)
    if wl.attn is not None:
        ac = shrink_attn(wl.attn, T=1, B=min(wl.attn.B, nb))
        ai = gen_attn(ac, seed, device="cpu", cid=wl.cid)
        f64 = lambda x: x[0].double().numpy()
        _CPU["attn"] = (f64(ai["trunk_k"]), f64(ai["trunk_v"]), f64(ai["q"]), f64(ai["k"]), f64(ai["v"]),
                        ai["anchors"][0].numpy(), ai["parent"][0].numpy(), ai["pos"][0].numpy())
        _CPU["nb"] = min(nb, ac.B)
    ctx = mp.get_context("fork")
    with ctx.Pool(1, initializer=_cpu_init) as pool:
        n1, t1 = 0, 0.0
        t0 = time.perf_counter()
        while t1 < budget_s / 2:
            pool.apply(_cpu_branch, (n1,))
            n1 += 1
            t1 = time.perf_counter() - t0
    per_branch = t1 / n1
    k = max(1, int(round(budget_s / 2 / per_branch)))
    with ctx.Pool(workers, initializer=_cpu_init) as pool:
        pool.map(_cpu_init_probe, range(workers), chunksize=1)  # workers up before the clock starts
        t0 = time.perf_counter()
        pool.map(_cpu_branch, range(workers * k), chunksize=1)
        tw = time.perf_counter() - t0
    rows_w = workers * k * lc.Wn
    return rows_w / tw, n1 * lc.Wn / t1, workers, n1 + workers * k, t1 + tw


def _cpu_init_probe(i):
    return i


def bench_qsa(sd, wl, seed, steps, warmup, dev, stream):
    """Block selection of a sparse-attention (QSA) target with
    branch-consistent indexer groups (specopd_qsa_select_fwd) on the
    workload's trunks and tree, timed on its own: the scoring step's
    counterpart for QSA layers.  Per launch, the scoring kernel forms one dot
    product of Di per candidate (every group complete at a node's position)
    and writes the candidate's fp32 score; the top-k kernel reads those
    scores back and writes k (index, score) pairs per node."""
    import numpy as np
    import torch
    from synthetic import gen_qsa
    qc = wl.qsa
    qi = gen_qsa(qc, seed, device=dev, cid=wl.cid)
    out = sd.qsa_select(qi, qc.topk, want_bkey=False)

    def call():
        sd.qsa_select(qi, qc.topk, ws=out["ws"], outs=out)

    for _ in range(max(1, warmup)):
        call()
    n = max(1, min(steps, 20))
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
    t5, c5 = sd.specopd_kernel_time(5)
    t6, c6 = sd.specopd_kernel_time(6)
    sd.specopd_kernel_timing(False)
    if sd.specopd_qsa_device_status(out["desc"], out["ws"]) != 0:
        raise SystemExit("QSA selection reported malformed branches")
    score_ms, topk_ms = t5 / c5, t6 / c6
    pos = qi["pos"].cpu().numpy().astype(np.int64)
    cand = float(((pos + 1) // 4).sum())
    rows = qc.T * qc.B * qc.Wn
    fl = 2.0 * qc.Di * cand
    score_bytes = 4.0 * cand + 2.0 * qc.T * (qc.L // 4) * qc.Di + 4.0 * rows * qc.Di
    topk_bytes = 4.0 * cand + 8.0 * rows * qc.topk
    ps = profile_summary(f"qsa_score_{wl.name}", QSA_SRC)
    pt = profile_summary(f"qsa_topk_{wl.name}", QSA_SRC)

    def roof(kind, ms, nbytes, prof, kernel):
        gbs = nbytes / (ms / 1e3) / 1e9
        t = _counter(prof, "hbm_bytes_per_launch")
        return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS,
                "traffic": None if t is None else t / (ms / 1e3) / 1e9, "traffic_unit": "GB/s",
                "traffic_bytes_per_launch": t, "valu_busy_pct": _counter(prof, "valu_busy_pct"),
                "kernel": kernel, "ms": ms, "alg_bytes_per_launch": nbytes}

    rs = roof("score", score_ms, score_bytes, ps, "qsa_score_kernel (specopd_qsa_select_fwd)")
    rs["mfma_tflops"] = fl / (score_ms / 1e3) / 1e12
    rs["mfma_frac"] = rs["mfma_tflops"] / BF16_PEAK_TFLOPS
    rs["alg_flops_per_launch"] = fl
    rt = roof("topk", topk_ms, topk_bytes, pt, "qsa_topk_kernel (specopd_qsa_select_fwd)")
    rt["candidates_per_s"] = cand / (topk_ms / 1e3)
    res = {
        "metric": "QSA branch rows/s (block selection, branch-consistent groups)",
        "value": rows / (call_ms / 1e3), "unit": "rows/s", "calls": n, "call_ms": call_ms,
        "candidates_per_row": cand / rows,
        "config": {"T": qc.T, "L": qc.L, "B": qc.B, "Wn": qc.Wn, "Di": qc.Di, "topk": qc.topk,
                   "dtype": qc.dtype},
        "roofline": rt if topk_ms >= score_ms else rs,
        "roofline_score": rs, "roofline_topk": rt,
    }
    del qi, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def bench_lmhead(sd, wl, seed, steps, warmup, dev, stream):
    """The LM head fused with E2E-TV (specopd_lmhead_e2etv_fwd_bwd) on the
    8B-layer shape: the branch rows' logits are formed from hidden states of
    4096 by the drafter's and the target's heads over the 151,936-entry
    vocabulary and never stored.  Algorithmic work: both logit matrices once,
    2 x 2 N V H FLOPs; the call forms the draft logits three times and the
    target logits twice (one per pass over the vocabulary; the gradient pass
    reads the indicator [q < p] from bits), 2.5 times that."""
    import torch
    from synthetic import gen_lmhead
    lc = wl.lmhead
    li = gen_lmhead(lc, seed, device=dev, cid=wl.cid)
    out = sd.lmhead_e2etv(li)

    def call():
        sd.lmhead_e2etv(li, ws=out["ws"], outs=out)

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
    tot, cnt = sd.specopd_kernel_time(7)
    sd.specopd_kernel_timing(False)
    if sd.specopd_lmhead_e2etv_device_status(out["desc"], out["ws"]) != 0:
        raise SystemExit("LM head + E2E-TV reported malformed branches")
    ms = tot / cnt
    N = lc.R * lc.Wn
    alg = 2.0 * 2.0 * N * lc.V * lc.H
    tf = alg / (ms / 1e3) / 1e12
    pl = profile_summary("lmhead_pass_layer8b", LMH_SRC)
    res = {
        "metric": "LM head + E2E-TV rows/s (logits never stored)", "value": N / (call_ms / 1e3),
        "unit": "rows/s", "calls": n, "call_ms": call_ms,
        "config": {"R": lc.R, "Wn": lc.Wn, "H": lc.H, "V": lc.V, "dtype": lc.dtype, "grad": "fp32"},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_PEAK_TFLOPS, "executed_tflops": 2.5 * tf,
                     "executed_frac": 2.5 * tf / BF16_PEAK_TFLOPS, "traffic": None,
                     "pass_b_hbm_bytes": _counter(pl, "hbm_bytes_per_launch"),
                     "pass_b_mfma_util_pct": _counter(pl, "mfma_util_pct"),
                     "kernel": "lmh_pass_kernel x3 + lse + scan (specopd_lmhead_e2etv_fwd_bwd)", "ms": ms,
                     "alg_flops_per_launch": alg},
    }
    del li, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def profile_summary(tag, src_files):
    """Key/value lines of profiles/<tag>.txt when the kernel sources it names
    are unchanged since it was taken (its source_sha256), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", tag + ".txt")
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
    return kv if kv.get("source_sha256") == h.hexdigest() else None


ATTN_SRC = ["speculative_decoding_drafter_amd/csrc/tree_attn_mfma.hip",
            "speculative_decoding_drafter_amd/csrc/device_common.h",
            "speculative_decoding_drafter_amd/csrc/internal.h",
            "speculative_decoding_drafter_amd/build.py"]
LOSS_SRC = ["speculative_decoding_drafter_amd/csrc/e2etv.hip",
            "speculative_decoding_drafter_amd/csrc/device_common.h",
            "speculative_decoding_drafter_amd/csrc/internal.h",
            "speculative_decoding_drafter_amd/build.py"]
GDN_SRC = ["speculative_decoding_drafter_amd/csrc/gdn.hip",
           "speculative_decoding_drafter_amd/csrc/device_common.h",
           "speculative_decoding_drafter_amd/csrc/internal.h",
           "speculative_decoding_drafter_amd/build.py"]


QSA_SRC = ["speculative_decoding_drafter_amd/csrc/qsa.hip",
           "speculative_decoding_drafter_amd/csrc/device_common.h",
           "speculative_decoding_drafter_amd/csrc/internal.h",
           "speculative_decoding_drafter_amd/build.py"]


LMH_SRC = ["speculative_decoding_drafter_amd/csrc/lmhead.hip",
           "speculative_decoding_drafter_amd/csrc/device_common.h",
           "speculative_decoding_drafter_amd/csrc/internal.h",
           "speculative_decoding_drafter_amd/build.py"]


def _counter(kv, key):
    try:
        return float(kv[key]) if kv is not None and key in kv else None
    except ValueError:
        return None


def measure(sd, wl, args, dev):
    """One workload: W warm-up steps, K eager steps with per-call events, K
    steps again with the library's kernel events, then K replays of the step
    captured as a HIP graph (the timed value unless --eager)."""
    import numpy as np
    import torch
    from synthetic import gen_attn, gen_loss

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
        # too, and the ratio converts the kernels' counters to bytes
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
    bad, deferred = sd.specopd_e2etv_device_status(ldesc, lws, with_deferred=True)
    if bad != 0:
        raise SystemExit("E2E-TV reported malformed branches")
    eager_ms_step = t_start.elapsed_time(t_end) / args.steps
    # The timed steps: the whole step (every kernel of both calls) captured
    # once as a HIP graph and replayed, which removes the host launch gaps
    # between its kernels; --eager times the plain calls instead.
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
        if ai is not None else eager_ms_step
    attn_ms = kern_ms[0] if kern_ms[0] else attn_call_ms
    loss_ms = kern_ms[1] if kern_ms[1] else loss_call_ms

    N = lc.N
    res = {
        "value": N / (ms_step / 1e3), "ms_per_step": ms_step,
        "graph": graph_ms_step is not None, "eager_ms_per_step": eager_ms_step,
        "deferred_rows": deferred,
    }
    if graph_note:
        res["graph_note"] = graph_note
    conf = {"workload": f"{wl.name} (workload {wl.cid})", "scored_rows": N,
            "loss": {"R": lc.R, "Wn": lc.Wn, "V": lc.V, "logits": lc.dtype, "grad": "f32"}}
    lb = loss_bytes(lc)
    loss_gbs = lb / (loss_ms / 1e3) / 1e9
    pl = profile_summary(f"e2etv_resident_{wl.name}", LOSS_SRC)
    t_loss = _counter(pl, "hbm_bytes_per_launch")
    roof_loss = {"bound": "hbm", "achieved": loss_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": loss_gbs / HBM_PEAK_GBS,
                 "traffic": None if t_loss is None else t_loss / (loss_ms / 1e3) / 1e9,
                 "traffic_bytes_per_launch": t_loss,
                 "valu_busy_pct": _counter(pl, "valu_busy_pct"),
                 "kernel": "e2etv_resident_kernel (specopd_e2etv_fwd_bwd)", "ms": loss_ms,
                 "call_ms": loss_call_ms, "alg_bytes_per_launch": lb}
    roofs = {"loss": roof_loss}
    if ai is not None:
        ac = wl.attn
        conf["attn"] = {"T": ac.T, "L": ac.L, "B": ac.B, "Wn": ac.Wn, "Hq": ac.Hq, "Hkv": ac.Hkv,
                        "D": ac.D, "dtype": ac.dtype}
        fl = attn_flops(ac, ai["anchors"].cpu().numpy())
        tf = fl / (attn_ms / 1e3) / 1e12
        peak = BF16_PEAK_TFLOPS if ac.dtype == "bf16" else FP32_PEAK_TFLOPS
        pa = profile_summary(f"tree_attn_mfma_{wl.name}", ATTN_SRC)
        t_attn = _counter(pa, "hbm_bytes_per_launch")
        roofs["attn"] = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                         "frac": tf / peak,
                         "traffic": None if t_attn is None else t_attn / (attn_ms / 1e3) / 1e9,
                         "traffic_unit": "GB/s", "traffic_bytes_per_launch": t_attn,
                         "mfma_util_pct": _counter(pa, "mfma_util_pct"),
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
    del ai, li, grad
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3,
                    help="1..5 (default: the batch of 8 trunks, the largest single-GPU workload)")
    ap.add_argument("--also", default="2,5",
                    help="other workloads measured the same way and reported under other_workloads "
                         "('' for none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=16.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the trunk-prefill measurement")
    ap.add_argument("--no-gdn", action="store_true", help="skip the GDN branch-replay measurement")
    ap.add_argument("--no-qsa", action="store_true", help="skip the QSA block-selection measurement")
    ap.add_argument("--no-lmhead", action="store_true",
                    help="skip the LM head + E2E-TV measurement (8B-layer shape)")
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

    from synthetic import WORKLOADS
    wl = WORKLOADS[args.workload]
    cpu = None
    if not args.no_cpu:
        # before anything touches the GPU: the oracle's workers are forked
        cpu = cpu_baseline(wl, args.seed, args.cpu_budget)

    import torch
    import speculative_decoding_drafter_amd as sd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.manual_seed(args.seed)
    m = measure(sd, wl, args, dev)
    res = {
        "metric": METRIC, "value": m.pop("value"), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": m.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.loss.dtype == "bf16" else "f32", "data": "synthetic",
    }
    res.update(m)
    if wl.attn is not None and not args.no_prefill:
        res["prefill"] = bench_prefill(sd, wl, args.seed, args.steps, args.warmup, dev,
                                       torch.cuda.current_stream())
    if wl.gdn is not None and not args.no_gdn:
        res["gdn"] = bench_gdn(sd, wl, args.seed, args.steps, args.warmup, dev, torch.cuda.current_stream())
    if wl.qsa is not None and not args.no_qsa:
        res["qsa"] = bench_qsa(sd, wl, args.seed, args.steps, args.warmup, dev, torch.cuda.current_stream())
    if not args.no_lmhead:
        lw = wl if wl.lmhead is not None else WORKLOADS[2]
        res["lmhead"] = bench_lmhead(sd, lw, args.seed, args.steps, args.warmup, dev, torch.cuda.current_stream())
    others = {}
    for c in [int(x) for x in args.also.split(",") if x.strip()]:
        if c == args.workload:
            continue
        o = measure(sd, WORKLOADS[c], args, dev)
        keep = ("value", "ms_per_step", "eager_ms_per_step", "deferred_rows", "roofline_attn",
                "roofline_loss")
        others[o["config"]["workload"]] = {k: o[k] for k in keep if k in o}
    if others:
        res["other_workloads"] = others
    if cpu is not None:
        v_all, v_one, workers, nb, secs = cpu
        res["cpu_baseline"] = {
            "value": v_all, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "value_one_core": v_one, "cpu_model": cpu_model(),
            "sample": f"{nb} whole branches of the {wl.name} configuration drawn on the host "
                      f"(tree attention of every node and head against the full trunk + the "
                      f"branch's E2E-TV forward/gradient rows), fp64 numpy, one BLAS thread per "
                      f"worker; one worker, then {workers} forked workers, {secs:.1f} s in all",
        }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
