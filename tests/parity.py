"""Comparison rules between the HIP library and the oracle.

Tolerances:
  * attention output: |gpu - ref| <= 1e-2 + 1e-2 |ref| elementwise (bf16 in,
    fp32 accumulate), plus relative L2 error <= 1e-2 as a second gate (the
    synthetic outputs are small, so the elementwise bound alone is loose);
    fp32 inputs: |gpu - ref| <= 2e-5 elementwise.
  * loss: relative error <= 1e-4, with an absolute floor of 1e-6 that only
    matters when the loss itself is ~0 (e.g. identical distributions): the
    kernel's alpha is an fp32 sum with absolute error ~1e-7, so a loss of
    exactly 0 comes out as ~1e-7 and a purely relative bound would be
    zero-width there.
  * alpha, prefix products: |gpu - ref| <= 1e-5.
  * gradient: |gpu - ref| <= 1e-5 elementwise, widened at exact-tie ambiguity
    (below), plus a relative L2 gate <= 1e-3 (5e-3 for a bf16 gradient) on the
    part of the error the tie envelope does not explain.

Gradient ties.  The gradient contains the indicator [q_u < p_u].  The GPU
decides it in fp32 from log2-probabilities, the oracle in fp64; where
|log p_u - log q_u| is within the fp32 error of that comparison the two may
legitimately differ.  That error bound (tie_tau) is per element: the kernel
forms lq = z log2(e) - lse2(z) and lp likewise with one fused multiply-add
each, so each carries at most half an fp32 ulp of its own magnitude plus the
error of its log-sum-exp (a relative error of the fp32 sum of exponentials,
taken as 1e-6 in log2 units); four ulps of the larger magnitude plus 2e-6,
converted to natural-log units, bounds the difference of the two -- about
7e-6 for typical rows (|lq| ~ 17 in log2 units), 2e-5 for the largest
logits here.  Each differing element moves grad[u] by |c| q_u and G by q_u,
i.e. every element of the row by |c| q_u q_v.  The envelope adds exactly
that much for every element u of an ambiguous set T:
    |c| * (q_u * sum_{v in T} q_v + [u in T] q_u).
Rows where that allowance exceeds a tenth of the row's gradient norm are
reported (printed with their allowance), not hidden.
Such ties are not rare with bf16 logits: when one token dominates each
distribution, log p - log q of every other token is a bf16-grid difference
minus a log-sum-exp difference that itself sits within ~1e-9 of a grid
value, so whole groups of tokens tie to ~1e-9.
Rows whose draft and target are bitwise identical are checked separately:
there both sides must give exactly zero.
"""

import numpy as np

ATTN_ATOL = 1e-2
ATTN_RTOL = 1e-2
ATTN_REL_L2 = 1e-2
ATTN_F32_ATOL = 2e-5
LOSS_RTOL = 1e-4
LOSS_ATOL_FLOOR = 1e-6
ALPHA_ATOL = 1e-5
GRAD_ATOL = 1e-5
GRAD_REL_L2 = 1e-3
GRAD_REL_L2_BF16 = 5e-3
LN2 = 0.6931471805599453
LOG2E = 1.4426950408889634


def tie_tau(lq, lp):
    """Per-element bound (natural-log units) on the error of the kernel's
    fp32 comparison of log2-probabilities; lq, lp natural-log probabilities
    (fp64, from the oracle)."""
    mag = np.maximum(np.abs(np.nan_to_num(lq, neginf=0.0)), np.abs(np.nan_to_num(lp, neginf=0.0)))
    ulp = np.spacing(np.float32(1.0)).astype(np.float64) * np.exp2(np.floor(np.log2(
        np.maximum(mag * LOG2E, 1e-30))))
    return LN2 * (4.0 * ulp + 2e-6)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def check_loss(gpu_loss, ref_loss, what="loss"):
    err = abs(float(gpu_loss) - float(ref_loss))
    assert err <= LOSS_RTOL * abs(ref_loss) + LOSS_ATOL_FLOOR, (
        f"{what}: gpu {gpu_loss!r} oracle {ref_loss!r} (abs err {err:.3e})")


def check_attention(gpu, ref, fp32=False, what="attention"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    if fp32:
        assert err.max() <= ATTN_F32_ATOL, f"{what}: max abs err {err.max():.3e}"
    bound = ATTN_ATOL + ATTN_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"
    r = rel_l2(gpu, ref)
    assert r <= ATTN_REL_L2, f"{what}: relative L2 {r:.3e}"
    return err.max(), r


def check_grad_rows(gpu, ref_grad, ref_margin, ref_q, coef, identical=None, bf16=False,
                    what="grad"):
    """gpu/ref_grad/ref_margin/ref_q: [n][V]; coef: [n] (grad_scale*dL/dalpha)."""
    gpu = np.asarray(gpu, np.float64)
    ref_grad = np.asarray(ref_grad, np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite"
    n = gpu.shape[0]
    resid = np.zeros_like(gpu)
    loose = []
    for i in range(n):
        if identical is not None and identical[i]:
            assert np.all(gpu[i] == 0.0), f"{what}: row {i} (target == draft) not exactly zero"
            continue
        with np.errstate(divide="ignore"):
            lq = np.log(ref_q[i])
        margin = np.nan_to_num(ref_margin[i], nan=0.0)
        tie = np.abs(margin) <= tie_tau(lq, lq + margin)
        env = np.zeros(gpu.shape[1])
        if tie.any():
            qt = float(ref_q[i][tie].sum())
            env = abs(coef[i]) * (ref_q[i] * qt + np.where(tie, ref_q[i], 0.0))
            gn = float(np.linalg.norm(ref_grad[i]))
            en = float(np.linalg.norm(env))
            if gn > 0 and en > 0.1 * gn:
                loose.append((i, int(tie.sum()), en / gn))
        atol = GRAD_ATOL if not bf16 else GRAD_ATOL + np.abs(ref_grad[i]) * 2.0 ** -8
        err = np.abs(gpu[i] - ref_grad[i])
        resid[i] = np.maximum(err - env, 0.0)
        bad = err > atol + env
        assert not bad.any(), (f"{what}: row {i}: {bad.sum()} elements out of tolerance, "
                               f"max err {err.max():.3e}")
    if loose:
        print(f"{what}: {len(loose)} of {n} rows have a tie allowance above 10% of their gradient "
              f"norm (row, tied elements, allowance/norm): {loose[:8]}", flush=True)
    keep = np.ones(n, bool) if identical is None else ~np.asarray(identical, bool)
    if keep.any():
        den = np.linalg.norm(ref_grad[keep])
        r = float(np.linalg.norm(resid[keep]) / (den if den > 0 else 1.0))
        lim = GRAD_REL_L2_BF16 if bf16 else GRAD_REL_L2
        assert r <= lim, f"{what}: relative L2 beyond the tie envelope {r:.3e}"
