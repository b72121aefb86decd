"""LM head fused with E2E-TV on the GPU through the C ABI, against the fp64
oracle (oracle.lmhead_e2etv: the two heads' logits, then E2E-TV).

Covered: every output (alpha, prefix products, loss, the whole logit
gradient) at reduced sizes -- chains, the forked tree and random trees,
hidden sizes 16 to 4096, vocabularies that end inside a 128-entry tile or a
64-entry chunk or are not a multiple of 4 (element-wise gradient stores),
row counts that end inside a 128-row tile, shared heads, siblings sharing a
target row, a global count and a gradient scale, the forward-only call --
malformed parent maps and target rows, determinism, and sampled branches at
the 8B-layer size (64 branches of 8, hidden 4096, vocabulary 151,936).

Tolerances are those of the E2E-TV call (tests/parity.py: alpha and prefix
1e-5, loss relative 1e-4, gradient 1e-5 plus the tie envelope).  Here the
kernel also forms the logits: fp32 sums of H exact bf16 products in 16-term
matrix-core steps, against the oracle's fp64 sums.  That moves a logit by
about 2^-24 sqrt(H/16) times the root of the sum of the squared products;
the tie envelope's comparison bound is widened by four times that for z
and for t, element by element, so an indicator [q < p] that the two
precisions may decide differently is accepted either way (the rule that an
integer decision is taken in each side's own precision)."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from parity import ALPHA_ATOL, check_loss, tie_tau
import parity
from synthetic import WORKLOADS, chain, gen_lmhead, shrink_lmhead

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.double().cpu().numpy()


def _logit_err(h, W2):
    """Per-element bound on the kernel's logit error (natural-log units of a
    logit), from the products' magnitudes (W2: the head squared)."""
    H = h.shape[-1]
    return 4.0 * 2.0 ** -24 * np.sqrt(H / 16.0) * np.sqrt((h * h) @ W2.T) + 1e-30


def _check_rows(out, inp, ref, rows, hd, Wd2, ht_rows, Wt2, what):
    """Gradient of the listed global rows against the oracle result `ref`
    (computed for those rows, in order)."""
    V = Wd2.shape[0]
    g = out["grad"].reshape(-1, V)[rows].double().cpu().numpy()
    ez = _logit_err(hd, Wd2)
    et = _logit_err(ht_rows, Wt2)
    resid = []
    for i in range(len(rows)):
        lq = np.log(np.maximum(ref["q"][i], 1e-300))
        margin = ref["margin"][i]
        # the comparison bound, widened by the logit errors of both sides
        tau = tie_tau(lq, lq + margin) + ez[i] + et[i]
        tie = np.abs(np.nan_to_num(margin)) <= tau
        env = np.zeros(V)
        if tie.any():
            qt = float(ref["q"][i][tie].sum())
            env = abs(ref["c"][i]) * (ref["q"][i] * qt + np.where(tie, ref["q"][i], 0.0))
        err = np.abs(g[i] - ref["grad"][i])
        bad = err > parity.GRAD_ATOL + env
        assert not bad.any(), f"{what}: row {rows[i]}: {bad.sum()} out of tolerance, max {err.max():.3e}"
        resid.append(np.maximum(err - env, 0.0))
    den = np.linalg.norm(ref["grad"])
    r = float(np.linalg.norm(np.stack(resid)) / (den if den > 0 else 1.0))
    assert r <= parity.GRAD_REL_L2, f"{what}: relative L2 beyond the envelope {r:.3e}"


def _oracle(inp, norm_count=None, grad_scale=1.0, branches=None):
    hd = _np(inp["h_draft"])
    R, Wn, H = hd.shape
    par = inp["parent"].cpu().numpy()
    tr = inp["target_row"].cpu().numpy()
    Wd, Wt, ht = _np(inp["w_draft"]), _np(inp["w_target"]), _np(inp["h_target"])
    bs = range(R) if branches is None else branches
    count = norm_count if norm_count else R * Wn
    res = {}
    for b in bs:
        r = oracle.lmhead_e2etv(hd[b:b + 1], Wd, ht, Wt, tr[b:b + 1], par[b:b + 1], norm_count=count,
                                grad_scale=grad_scale)
        z = hd[b] @ Wd.T
        q = np.exp(z - oracle.logsumexp(z))
        r["q"] = q
        r["c"] = r["dL_dalpha"][0]  # grad_scale included
        res[b] = r
    return res


def _run(inp, norm_count=0.0, grad_scale=1.0, grad=True):
    out = sd.lmhead_e2etv(inp, grad=grad, norm_count=norm_count, grad_scale=grad_scale)
    torch.cuda.synchronize()
    return out


def _check_all(inp, out, norm_count=None, grad_scale=1.0, branches=None, grad=True):
    res = _oracle(inp, norm_count, grad_scale, branches)
    hd = _np(inp["h_draft"])
    R, Wn, H = hd.shape
    Wd, Wt, ht = _np(inp["w_draft"]), _np(inp["w_target"]), _np(inp["h_target"])
    tr = inp["target_row"].cpu().numpy()
    al = out["alpha"].double().cpu().numpy()
    pr = out["prefix"].double().cpu().numpy()
    Wd2, Wt2 = (Wd * Wd, Wt * Wt) if grad else (None, None)
    for b, r in res.items():
        assert np.abs(al[b] - r["alpha"][0]).max() <= ALPHA_ATOL, f"alpha branch {b}"
        assert np.abs(pr[b] - r["prefix"][0]).max() <= ALPHA_ATOL, f"prefix branch {b}"
        if grad:
            ref = {"grad": r["grad"][0], "margin": r["margin"][0], "q": r["q"], "c": r["c"]}
            _check_rows(out, inp, ref, [b * Wn + j for j in range(Wn)], hd[b], Wd2, ht[tr[b]], Wt2,
                        f"grad branch {b}")
    loss = out["loss"].cpu().numpy()
    count = norm_count if norm_count else R * Wn
    assert loss[2] == count
    if branches is None:
        numer = sum(r["numer"] for r in res.values())
        check_loss(loss[0], 1.0 - numer / count)
        assert abs(loss[1] - numer) <= 1e-5 * max(1.0, numer)
    # the loss is the sum of the kernel's own prefix products either way
    assert abs(loss[1] - pr.sum()) <= 1e-4 * max(1.0, abs(loss[1]))


@pytest.mark.parametrize("kw", [
    dict(L=100, P=20, R=3, H=64, V=1000),                      # chains of 8
    dict(L=60, P=10, R=5, H=256, V=1031),                      # V not a multiple of 4
    dict(L=300, P=40, R=17, H=128, V=130),                     # 136 rows; V ends inside a tile
    dict(L=40, P=5, R=2, H=16, V=65, parent=(-1, 0, 1, 2, 3, 4, 5, 3, 7, 8)),   # forked tree
    dict(L=50, P=10, R=2, H=4096, V=3000),                     # the 8B hidden size
])
def test_matches_oracle(gpu_ok, kw):
    cfg = shrink_lmhead(WORKLOADS[2].lmhead, **kw)
    inp = gen_lmhead(cfg, 5, device=DEV, cid=2)
    out = _run(inp)
    assert sd.specopd_lmhead_e2etv_device_status(out["desc"], out["ws"]) == 0
    _check_all(inp, out)


def test_random_trees_shared_head_count_and_scale(gpu_ok):
    rng = np.random.default_rng(7)
    Wn = 13
    cfg = shrink_lmhead(WORKLOADS[2].lmhead, L=80, P=10, R=4, H=128, V=777, parent=chain(Wn)[0])
    inp = gen_lmhead(cfg, 8, device=DEV, cid=2)
    par = np.stack([[-1] + [int(rng.integers(-1, j)) for j in range(1, Wn)] for _ in range(cfg.R)])
    inp["parent"] = torch.from_numpy(par.astype(np.int32)).to(DEV)
    anch = inp["anchors"].cpu().numpy()
    rows = np.array([[anch[r] if par[r, j] < 0 else cfg.L + r * Wn + par[r, j] for j in range(Wn)]
                     for r in range(cfg.R)], np.int32)
    inp["target_row"] = torch.from_numpy(rows).to(DEV)
    inp["w_target"] = inp["w_draft"]  # one head for both models
    out = _run(inp, norm_count=1000.0, grad_scale=0.5)
    _check_all(inp, out, norm_count=1000.0, grad_scale=0.5)


def test_forward_only_and_determinism(gpu_ok):
    cfg = shrink_lmhead(WORKLOADS[2].lmhead, L=200, P=20, R=6, H=256, V=2000)
    inp = gen_lmhead(cfg, 9, device=DEV, cid=2)
    a = _run(inp)
    b = _run(inp)
    f = _run(inp, grad=False)
    for k in ("alpha", "prefix", "loss", "grad"):
        assert torch.equal(a[k], b[k]), k
    for k in ("alpha", "prefix", "loss"):
        assert torch.equal(a[k], f[k]), k


def test_malformed_branches_and_rows_are_flagged(gpu_ok):
    cfg = shrink_lmhead(WORKLOADS[2].lmhead, L=100, P=20, R=4, H=64, V=500)
    inp = gen_lmhead(cfg, 10, device=DEV, cid=2)
    good = _run(inp)
    par = inp["parent"].clone()
    par[1, 3] = 5                                    # parent after its child
    tr = inp["target_row"].clone()
    tr[2, 0] = inp["h_target"].shape[0]              # target row outside h_target
    bad = dict(inp, parent=par, target_row=tr)
    out = _run(bad)
    assert sd.specopd_lmhead_e2etv_device_status(out["desc"], out["ws"]) == 2
    for b in (1, 2):
        assert torch.isnan(out["alpha"][b]).any() and torch.isnan(out["prefix"][b]).any()
    assert np.isnan(out["loss"][0].item())
    for b in (0, 3):
        assert torch.equal(out["alpha"][b], good["alpha"][b])
        assert torch.equal(out["grad"][b], good["grad"][b])


def test_full_size_sampled_branches(gpu_ok):
    cfg = WORKLOADS[2].lmhead
    inp = gen_lmhead(cfg, 0, device=DEV, cid=2)
    out = _run(inp)
    assert sd.specopd_lmhead_e2etv_device_status(out["desc"], out["ws"]) == 0
    _check_all(inp, out, branches=[0, 17, 63])
