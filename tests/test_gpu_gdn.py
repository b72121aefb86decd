"""GDN branch replay on the GPU through the C ABI against the fp64 oracle.

Every output element at sizes the oracle finishes in seconds (trunk lengths
that are and are not multiples of the checkpoint interval, anchors on both
sides of a checkpoint, a trunk shorter than one interval, chains and the
forked tree, head sizes 64 and 128, bf16 and fp32 inputs), gates small
enough to exercise the state's rescaling and gates of zero, malformed
branches, sampled branches at the full workload sizes, and the replay
against a full sequential recomputation from checkpoints the oracle's own
trunk pass produced (jaehun.me review §3.2(c), Fig. 5; §3.2 consistency).

Tolerance.  The kernel keeps the state in fp32 as g * St (one scale per
head) and forms each S k and S q as a sum of D fp32 products in a fixed
order; the oracle runs in fp64.  Each update adds a few units of fp32
rounding (2^-24 ~ 6e-8) relative to the state's row norms (order one with
unit keys and values of order one), and a branch runs at most C - 1 + Wn
updates (about 80), so the state's error stays near 80 * 4 * 6e-8 ~ 2e-5
relative in the worst case and far less on average (errors of either sign);
an output reads the state against a query of norm ~sqrt(D).  Measured: at
most 1.6e-6 absolute against outputs up to ~10.  The check allows 2e-5 +
2e-5 |ref| per element."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from synthetic import FORK_PARENT, WORKLOADS, chain, gen_gdn, shrink_gdn

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL = 2e-5
RTOL = 2e-5


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _ref(inp, branches=None, C=64):
    return oracle.gdn_replay(_np(inp["ckpt"]), _np(inp["trunk_k"]), _np(inp["trunk_v"]),
                             _np(inp["trunk_gate"]), _np(inp["trunk_beta"]), inp["anchors"].cpu().numpy(),
                             inp["parent"].cpu().numpy(), _np(inp["q"]), _np(inp["k"]), _np(inp["v"]),
                             _np(inp["gate"]), _np(inp["beta"]), C=C, branches=branches)


def _check(got, ref, what=""):
    got = got.cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"


def _run(inp, C=64):
    out, desc, ws = sd.gdn_replay(inp, C=C)
    torch.cuda.synchronize()
    return out, desc, ws


@pytest.mark.parametrize("cid,kw", [
    (3, dict(T=2, L=300, P=64, B=6, H=3, D=128, dtype="bf16")),            # chains of 16, ragged trunk
    (3, dict(T=1, L=256, P=16, B=5, H=2, D=64, dtype="bf16")),             # D=64, L a multiple of C
    (5, dict(T=1, L=200, P=30, B=6, H=2, D=128, dtype="bf16")),            # forked tree
    (2, dict(T=2, L=130, P=10, B=4, H=2, D=128, dtype="f32")),             # fp32 inputs, chains of 8
    (5, dict(T=1, L=150, P=20, B=4, H=2, D=64, dtype="f32")),              # fp32, fork, D=64
])
def test_reduced_workloads(gpu_ok, cid, kw):
    cfg = shrink_gdn(WORKLOADS[cid].gdn, **kw)
    inp = gen_gdn(cfg, 3, device=DEV, cid=cid)
    out, desc, ws = _run(inp)
    assert sd.specopd_gdn_device_status(desc, ws) == 0
    _check(out, _ref(inp), f"wl{cid} {kw}")


def test_anchors_around_checkpoints(gpu_ok):
    """Anchors at 0, on both sides of each checkpoint and at the trunk's end:
    no replay (a = 64m - 1), one token, 63 tokens, and the zero state."""
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=200, P=0, B=10, H=2, D=128, parent=chain(5)[0])
    inp = gen_gdn(cfg, 5, device=DEV, cid=3)
    inp["anchors"] = torch.tensor([[0, 1, 62, 63, 64, 65, 127, 128, 191, 199]], dtype=torch.int32, device=DEV)
    out, desc, ws = _run(inp)
    _check(out, _ref(inp), "anchors around checkpoints")


def test_trunk_shorter_than_one_interval(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=2, L=40, P=0, B=4, H=2, D=64, parent=chain(6)[0])
    inp = gen_gdn(cfg, 6, device=DEV, cid=3)
    assert inp["ckpt"].shape[1] == 0
    out, desc, ws = _run(inp)  # no checkpoint pointer passed
    _check(out, _ref(inp), "no checkpoints")


def test_small_and_zero_gates(gpu_ok):
    """Gates of 1e-3 drive the running scale below 2^-30 within a few tokens
    (the state is rescaled); a gate of zero erases the state."""
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=180, P=0, B=6, H=2, D=128, parent=chain(9)[0])
    inp = gen_gdn(cfg, 7, device=DEV, cid=3)
    inp["trunk_gate"][:, ::3] = 1e-3
    inp["gate"][:, :, 2] = 0.0
    inp["gate"][:, :, 5] = 1e-3
    out, desc, ws = _run(inp)
    _check(out, _ref(inp), "small and zero gates")


def test_trunk_pass_checkpoints_replay_equals_full_recomputation(gpu_ok):
    """With checkpoints from the oracle's own trunk pass, every node's output
    equals reading one sequential recurrence over its whole history."""
    cfg = shrink_gdn(WORKLOADS[5].gdn, T=1, L=160, P=0, B=5, H=2, D=64, dtype="f32")
    inp = gen_gdn(cfg, 8, device=DEV, cid=5)
    ck = oracle.trunk_checkpoints(_np(inp["trunk_k"][0]), _np(inp["trunk_v"][0]), _np(inp["trunk_gate"][0]),
                                  _np(inp["trunk_beta"][0]), 64)
    inp["ckpt"] = torch.from_numpy(ck[None]).float().to(DEV).contiguous()
    out, desc, ws = _run(inp)
    got = out.cpu().numpy().astype(np.float64)
    par = FORK_PARENT
    anch = inp["anchors"].cpu().numpy()
    tk, tv, ta, tb = (_np(inp[n][0]) for n in ("trunk_k", "trunk_v", "trunk_gate", "trunk_beta"))
    q, k, v, g, be = (_np(inp[n][0]) for n in ("q", "k", "v", "gate", "beta"))
    for b in range(cfg.B):
        a = int(anch[0, b])
        for j in range(len(par)):
            path, x = [], j
            while x >= 0:
                path.append(x)
                x = par[x]
            path = path[::-1]
            for h in range(cfg.H):
                S = oracle.run_tokens(np.zeros((64, 64)),
                                      np.concatenate([tk[:a + 1, h], k[b, path, h]]),
                                      np.concatenate([tv[:a + 1, h], v[b, path, h]]),
                                      np.concatenate([ta[:a + 1, h], g[b, path, h]]),
                                      np.concatenate([tb[:a + 1, h], be[b, path, h]]))[-1]
                ref = S @ q[b, j, h]
                assert np.all(np.abs(got[0, b, j, h] - ref) <= ATOL + RTOL * np.abs(ref)), (b, j, h)


def test_malformed_branches_are_flagged(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=150, P=0, B=5, H=2, D=128, parent=chain(6)[0])
    inp = gen_gdn(cfg, 9, device=DEV, cid=3)
    inp["anchors"][0, 1] = 150           # outside the trunk
    inp["parent"][0, 3, 4] = 4           # a node that is its own parent
    out, desc, ws = _run(inp)
    assert sd.specopd_gdn_device_status(desc, ws) == 2
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[0, 1])) and np.all(np.isnan(got[0, 3]))
    good = [(0, 0), (0, 2), (0, 4)]
    ref = _ref(inp, branches=good)
    for t, b in good:
        _check(got[t, b], ref[t, b], f"branch {b}")
    # the next call on the same workspace starts its count afresh
    inp["anchors"][0, 1] = 10
    inp["parent"][0, 3, 4] = 3
    out, desc, ws2 = sd.gdn_replay(inp, ws=ws)
    assert sd.specopd_gdn_device_status(desc, ws2) == 0


def _branch_ref(inp, t, b, C):
    """One branch's outputs [Wn][H][D] from the oracle's pieces, copying to the
    host only the checkpoint and the trunk tokens the branch replays."""
    a = int(inp["anchors"][t, b])
    c, t0 = oracle.replay_span(a, C)
    H, D = inp["q"].shape[3], inp["q"].shape[4]
    S0 = _np(inp["ckpt"][t, c]) if c >= 0 else np.zeros((H, D, D))
    tk, tv = _np(inp["trunk_k"][t, t0:a + 1]), _np(inp["trunk_v"][t, t0:a + 1])
    ta, tb = _np(inp["trunk_gate"][t, t0:a + 1]), _np(inp["trunk_beta"][t, t0:a + 1])
    par = inp["parent"][t, b].cpu().numpy()
    q, k, v = _np(inp["q"][t, b]), _np(inp["k"][t, b]), _np(inp["v"][t, b])
    g, be = _np(inp["gate"][t, b]), _np(inp["beta"][t, b])
    out = np.empty((len(par), H, D))
    for h in range(H):
        Sa = oracle.run_tokens(S0[h], tk[:, h], tv[:, h], ta[:, h], tb[:, h])[-1] if a >= t0 else S0[h]
        st = []
        for j, p in enumerate(par):
            Sj = oracle.gated_delta_update(Sa if p < 0 else st[p], k[j, h], v[j, h], g[j, h], be[j, h])
            st.append(Sj)
            out[j, h] = oracle.gdn_read(Sj, q[j, h])
    return out


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_full_size_sampled_branches(gpu_ok, cid):
    cfg = WORKLOADS[cid].gdn
    inp = gen_gdn(cfg, 0, device=DEV, cid=cid)
    out, desc, ws = _run(inp)
    assert sd.specopd_gdn_device_status(desc, ws) == 0
    rng = np.random.default_rng(cid)
    picks = sorted({(int(rng.integers(cfg.T)), int(rng.integers(cfg.B))) for _ in range(3)})
    anch = inp["anchors"].cpu().numpy()
    picks.append((0, int(((anch[0] + 1) % cfg.C).argmax())))  # the longest replay of trunk 0
    for t, b in picks:
        _check(out[t, b], _branch_ref(inp, t, b, cfg.C), f"wl{cid} branch {(t, b)}")


def test_deterministic(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=2, L=400, P=64, B=16, H=4, D=128)
    inp = gen_gdn(cfg, 11, device=DEV, cid=3)
    a, _, ws = _run(inp)
    b, _, _ = sd.gdn_replay(inp, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kernel_timing_records_each_call(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=200, P=16, B=8, H=2, D=128)
    inp = gen_gdn(cfg, 12, device=DEV, cid=3)
    out, desc, ws = _run(inp)
    sd.specopd_kernel_timing(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(2):
        sd.gdn_replay(inp, ws=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms, n = sd.specopd_kernel_time(3)
    sd.specopd_kernel_timing(False)
    assert n == 2 and 0 < ms <= e0.elapsed_time(e1) * 1.05
