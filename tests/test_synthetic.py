"""The seeded generator: determinism, shapes, structure of anchors / trees /
row classes.  CPU only, at reduced sizes."""

import numpy as np
import torch

import oracle
from synthetic import (WORKLOADS, gen_attn, gen_loss, shrink_attn, shrink_loss, FORK_PARENT,
                       FORK_DEPTH, stress_classes)


def test_workload_table_matches_descriptions():
    w = WORKLOADS
    assert w[1].attn.L == 64 and w[1].attn.B == 4 and w[1].attn.Wn == 4 and w[1].attn.D == 64
    assert w[1].loss.N == 16 and w[1].loss.V == 1000
    assert w[2].attn.rows == 512 and w[2].loss.N == 512
    assert w[3].attn.rows == 16384 and w[3].loss.N == 16384
    assert w[4].attn is None and w[4].loss.N == 7168
    assert w[5].attn.rows == 5120 and w[5].loss.N == 5120
    # the forked tree: every root-to-leaf path has 7 tokens
    assert list(oracle.tree_depths(FORK_PARENT)) == list(FORK_DEPTH)
    leaves = [j for j in range(10) if j not in oracle.new_score_rows(FORK_PARENT)]
    assert all(len(oracle.walk_ancestors(FORK_PARENT, j)) == 7 for j in leaves)


def test_attn_determinism_and_structure():
    cfg = shrink_attn(WORKLOADS[2].attn, L=300, P=64, B=7)
    a = gen_attn(cfg, seed=3, cid=2)
    b = gen_attn(cfg, seed=3, cid=2)
    c = gen_attn(cfg, seed=4, cid=2)
    for key in a:
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["q"], c["q"])
    assert a["trunk_k"].shape == (1, 300, 8, 128) and a["trunk_k"].dtype == torch.bfloat16
    assert a["q"].shape == (1, 7, 8, 32, 128)
    anch = a["anchors"].numpy()
    assert anch.min() >= 64 and anch.max() < 299 and len(set(anch[0].tolist())) == 7
    for bb in range(7):
        oracle.check_positions(anch[0, bb], a["parent"][0, bb].numpy(), a["pos"][0, bb].numpy())
    x = a["q"].float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1) < 0.02


def test_fork_tree_positions():
    cfg = shrink_attn(WORKLOADS[5].attn, L=200, P=50, B=3, Hq=6, Hkv=1, D=8)
    a = gen_attn(cfg, seed=0, cid=5)
    for bb in range(3):
        oracle.check_positions(a["anchors"][0, bb].item(), a["parent"][0, bb].numpy(), a["pos"][0, bb].numpy())


def test_loss_recipes():
    cfg = shrink_loss(WORKLOADS[3].loss, R=4, V=5000)
    d = gen_loss(cfg, seed=0, cid=3)
    z, t = d["draft"].float().reshape(-1), d["target"].float().reshape(-1)
    assert abs(z.std().item() - 3) < 0.1 and abs(t.std().item() - 3) < 0.1
    r = np.corrcoef(z.numpy(), t.numpy())[0, 1]
    assert abs(r - 0.8) < 0.02
    cfg = shrink_loss(WORKLOADS[4].loss, R=16, V=3000)
    d = gen_loss(cfg, seed=1, cid=4, chunk_rows=20)
    cls = stress_classes(cfg, 1, 4)
    assert (cls == 0).sum() == 56 and (cls == 1).sum() == 28 and (cls == 2).sum() == 28
    z = d["draft"].reshape(-1, 3000)
    t = d["target"].reshape(-1, 3000)
    for n in range(cfg.N):
        if cls[n] == 0:
            assert torch.equal(z[n], t[n])
        elif cls[n] == 1:
            assert z[n].float().argmax() != t[n].float().argmax()
            assert z[n].float().max() > 25 and t[n].float().max() > 25
    res = oracle.e2etv(d["draft"], d["target"], d["parent"], with_grad=False)
    al = res["alpha"].reshape(-1)
    np.testing.assert_allclose(al[cls == 0], 1.0, atol=1e-12)
    assert np.all(al[cls == 1] < 1e-6)
    d2 = gen_loss(cfg, seed=1, cid=4, chunk_rows=20)
    assert torch.equal(d["draft"], d2["draft"]) and torch.equal(d["target"], d2["target"])
