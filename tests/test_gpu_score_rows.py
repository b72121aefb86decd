"""Which attention row scores which branch token, on the GPU.

jaehun.me review §3.2(a) and Fig. 3 (rustineverything.app summary §2.2): a
row's output predicts the token after it, so a branch token's target
distribution comes from its parent's row, or from the anchor's trunk row for
a token attached to the anchor; siblings share their parent's row.
specopd_score_rows writes that row index for every node, and
specopd_e2etv_fwd_bwd gathers the target logits through it.  Checked against
the Fig. 3 worked example, against oracle.score_row_source on forked trees,
and end to end: prefill rows and tree-attention rows -> (a linear read-out
standing in for the rest of the target model, test plumbing) -> E2E-TV with
the gather, against oracle.e2etv on targets gathered by the oracle."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from conftest import golden_dict
from parity import ALPHA_ATOL, check_grad_rows, check_loss
from synthetic import FORK_PARENT, WORKLOADS, gen_attn, gen_prefill, shrink_attn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_rows(anchors, parent, L):
    T, B, Wn = parent.shape
    rows = np.empty((T, B, Wn), np.int64)
    for t in range(T):
        for b in range(B):
            for j in range(Wn):
                kind, idx = oracle.score_row_source(anchors[t, b], parent[t, b], j)
                rows[t, b, j] = t * L + idx if kind == "trunk" else T * L + (t * B + b) * Wn + idx
    return rows


def test_fig3_toy_tree_rows(gpu_ok):
    g = golden_dict("fig3_toy_tree.txt")
    L = int(g["L"][0][0])
    anchors = np.array([[int(a[1]) for a in g["anchor"]]], np.int32)
    B = anchors.shape[1]
    nodes = g["node"]
    Wn = max(int(n[1]) for n in nodes) + 1
    parent = np.zeros((1, B, Wn), np.int32)
    for n in nodes:
        parent[0, int(n[0]), int(n[1])] = int(n[3])
    rows = sd.score_rows(torch.tensor(anchors, device=DEV), torch.tensor(parent, device=DEV), L)
    got = rows.cpu().numpy()
    for b, j, kind, idx in g["score"]:
        b, j, idx = int(b), int(j), int(idx)
        want = idx if kind == "trunk" else L + b * Wn + idx
        assert got[0, b, j] == want, (b, j, kind, idx, got[0, b, j])
    assert np.array_equal(got, _oracle_rows(anchors, parent, L))


def test_rows_of_random_trees_and_malformed_branches(gpu_ok):
    rng = np.random.default_rng(21)
    T, B, Wn, L = 3, 37, 23, 500
    anchors = rng.integers(0, L, size=(T, B)).astype(np.int32)
    parent = np.empty((T, B, Wn), np.int32)
    for t in range(T):
        for b in range(B):
            parent[t, b] = [-1] + [int(rng.integers(-1, j)) for j in range(1, Wn)]
    bad = parent.copy()
    bad[1, 5, 7] = 7           # self-parent
    bad[2, 0, 3] = 9           # parent after child
    anc_bad = anchors.copy()
    anc_bad[0, 11] = L         # anchor outside the trunk
    rows = sd.score_rows(torch.tensor(anc_bad, device=DEV), torch.tensor(bad, device=DEV), L).cpu().numpy()
    ref = _oracle_rows(anchors, parent, L)
    for (t, b) in ((1, 5), (2, 0), (0, 11)):
        assert np.all(rows[t, b] == -1)
        ref[t, b] = -1
    assert np.array_equal(rows, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_tree_and_loss_chained_on_forked_trees(gpu_ok, dtype):
    cfg = shrink_attn(WORKLOADS[5].attn, T=2, L=300, P=60, B=4, Hq=4, Hkv=2, D=64, dtype=dtype)
    Wn = cfg.Wn
    assert cfg.parent == FORK_PARENT
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # trunk rows from the prefill, branch rows from tree attention on its cache
    pre = gen_prefill(cfg, 3, device=DEV, cid=5)
    pout, ck, cv, _, _ = sd.prefill(pre["q"], pre["k"], pre["v"])
    br = gen_attn(cfg, 3, device=DEV, cid=5)
    br["trunk_k"], br["trunk_v"] = ck, cv
    bout, desc, ws = sd.tree_attn(br)
    torch.cuda.synchronize()
    assert sd.specopd_tree_attn_device_status(desc, ws) == 0
    hidden = torch.cat([pout.reshape(cfg.T * cfg.L, -1), bout.reshape(cfg.T * cfg.B * Wn, -1)]).float()
    # a linear read-out to a vocabulary of 4099 (test plumbing, not the path)
    V = 4099
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    W = torch.randn(hidden.shape[1], V, generator=g, device=DEV) * 2.0
    target = (hidden @ W).to(dt).contiguous()                      # [rows][V]
    draft = (target[torch.randint(0, target.shape[0], (cfg.T * cfg.B * Wn,), generator=g, device=DEV)]
             .float() + torch.randn(cfg.T * cfg.B * Wn, V, generator=g, device=DEV)).to(dt)
    draft = draft.reshape(cfg.T * cfg.B, Wn, V).contiguous()
    rows = sd.score_rows(br["anchors"], br["parent"], cfg.L)
    parent = br["parent"].reshape(cfg.T * cfg.B, Wn).contiguous()
    out = sd.e2etv(draft, target, parent, target_row=rows.reshape(cfg.T * cfg.B, Wn).contiguous())
    torch.cuda.synchronize()
    assert sd.specopd_e2etv_device_status(out["desc"], out["ws"]) == 0
    # the oracle: its own row map, the gathered targets, the plain loss
    ref_rows = _oracle_rows(br["anchors"].cpu().numpy(), br["parent"].cpu().numpy(), cfg.L)
    assert np.array_equal(rows.cpu().numpy(), ref_rows)
    tg = target.cpu()[torch.tensor(ref_rows.reshape(-1))].reshape(cfg.T * cfg.B, Wn, V)
    ref = oracle.e2etv(draft.cpu(), tg, parent.cpu())
    assert np.abs(out["alpha"].cpu().double().numpy() - ref["alpha"]).max() <= ALPHA_ATOL
    assert np.abs(out["prefix"].cpu().double().numpy() - ref["prefix"]).max() <= ALPHA_ATOL
    check_loss(out["loss"][0].item(), ref["loss"])
    n = cfg.T * cfg.B * Wn
    q = np.exp(oracle.log_softmax(draft.reshape(n, V).cpu().double().numpy()))
    check_grad_rows(out["grad"].reshape(n, V).cpu().numpy(), ref["grad"].reshape(n, V),
                    ref["margin"].reshape(n, V), q, ref["dL_dalpha"].reshape(n))
    # siblings (nodes 4 and 7 both hang off node 3) read the same target row
    r = rows.cpu().numpy()
    assert np.all(r[:, :, 4] == r[:, :, 7])


def test_target_row_outside_the_matrix_flags_its_branch(gpu_ok):
    R, Wn, V = 4, 3, 4096
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    target = torch.randn(7, V, generator=g, device=DEV).bfloat16()
    draft = torch.randn(R, Wn, V, generator=g, device=DEV).bfloat16()
    parent = torch.tensor([[-1, 0, 1]] * R, dtype=torch.int32, device=DEV)
    tr = torch.tensor([[0, 1, 2], [3, 4, 5], [6, 7, 0], [1, 2, 3]], dtype=torch.int32, device=DEV)
    out = sd.e2etv(draft, target, parent, target_row=tr)
    assert sd.specopd_e2etv_device_status(out["desc"], out["ws"]) == 1
    a = out["alpha"].cpu().numpy()
    assert np.all(np.isnan(a[2])) and np.all(np.isfinite(a[[0, 1, 3]]))
    assert torch.isnan(out["grad"][2]).all() and torch.isfinite(out["grad"][[0, 1, 3]]).all()
