"""Shapes and value recipes of the five synthetic workloads.

These are the workload descriptions only: sizes, tree shapes, dtypes and the
distributions values are drawn from.  Nothing here computes any part of the
scoring method.  The generator in ``synthetic.gen`` turns a config plus a seed
into tensors; both the CPU oracle and the GPU library consume those tensors.

Tree shapes.  A branch is a list of ``Wn`` nodes; ``parent[j]`` is -1 for the
node attached to the anchor and otherwise an earlier node index, and
``depth[j]`` is the node's offset from the anchor (the semantic position of
node j is anchor + 1 + depth[j]).  Both tuples are literal input structure:
chains have parent j-1 and depth j; the forked tree used by the long-context
workload is a chain of offsets 0..3 that splits into two sub-branches of
offsets 4..6 (ten nodes, every root-to-leaf path seven tokens long).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


def chain(w: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Parent map and depths of a chain branch of ``w`` nodes."""
    return tuple([-1] + list(range(w - 1))), tuple(range(w))


# Chain of offsets 0..3, then two sub-branches of offsets 4..6.
FORK_PARENT = (-1, 0, 1, 2, 3, 4, 5, 3, 7, 8)
FORK_DEPTH = (0, 1, 2, 3, 4, 5, 6, 4, 5, 6)


@dataclass(frozen=True)
class AttnConfig:
    """Tree-attention workload: T trunks of length L (first P tokens prompt),
    B anchored branches per trunk, each a tree of Wn nodes."""

    T: int
    L: int
    P: int
    B: int
    parent: Tuple[int, ...]
    depth: Tuple[int, ...]
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" | "bf16"
    rope_base: float = 10000.0

    @property
    def Wn(self) -> int:
        return len(self.parent)

    @property
    def rows(self) -> int:
        """Scored branch rows T*B*Wn (each across Hq heads)."""
        return self.T * self.B * self.Wn


@dataclass(frozen=True)
class LossConfig:
    """E2E-TV workload: R branches of Wn nodes, vocabulary V.

    recipe:
      "indep"  draft, target independent N(0, sd^2)
      "noise"  draft ~ N(0, 1), target = draft + N(0, 1)
      "rho"    draft = sd*e1, target = rho*draft + sd*sqrt(1-rho^2)*e2
      "stress" half the rows target == draft bitwise, a quarter
               disjoint one-hot-peaked (+peak at distinct tokens), a quarter
               "noise"; rows assigned by a seeded permutation
    """

    R: int
    parent: Tuple[int, ...]
    V: int
    dtype: str
    recipe: str
    sd: float = 1.0
    rho: float = 0.0
    peak: float = 32.0

    @property
    def Wn(self) -> int:
        return len(self.parent)

    @property
    def N(self) -> int:
        return self.R * self.Wn


@dataclass(frozen=True)
class GdnConfig:
    """Linear-attention (GDN) branch replay workload: T trunks of length L
    (first P tokens prompt) with a recurrent state checkpoint every C trunk
    tokens, B anchored branches per trunk (each a tree of Wn nodes), H heads
    with key and value size D.

    Value laws: keys (trunk and branch) uniform on the unit sphere (Gaussian
    draws scaled to unit length), values and queries N(0, 1), all rounded to
    the dtype; decay gates uniform in [gate_lo, 1); write strengths uniform in
    [0.05, 0.95); checkpoint states N(0, state_sd^2) in fp32."""

    T: int
    L: int
    P: int
    B: int
    parent: Tuple[int, ...]
    H: int
    D: int
    dtype: str  # "f32" | "bf16" (queries, keys, values)
    C: int = 64
    gate_lo: float = 0.85
    state_sd: float = 0.1

    @property
    def Wn(self) -> int:
        return len(self.parent)

    @property
    def NC(self) -> int:
        """Checkpoints per trunk (state after every C tokens)."""
        return self.L // self.C


@dataclass(frozen=True)
class QsaConfig:
    """Sparse-attention (QSA) block-selection workload: T trunks of length L
    (first P tokens prompt), B anchored branches per trunk (each a tree of Wn
    nodes), indexer key size Di, topk groups of 4 tokens kept per node.

    Value laws: raw indexer keys and indexer queries N(0, 1) in bf16; the
    RMSNorm gain 1 + N(0, 0.1^2) in fp32; the trunk's group-key cache N(0, 1)
    in bf16 where a test does not build it from the raw keys (a compressed key
    has unit root-mean-square times the gain, and a Gaussian vector is
    unchanged in law by the rotation, so the draw has the cache's scale)."""

    T: int
    L: int
    P: int
    B: int
    parent: Tuple[int, ...]
    Di: int
    topk: int
    dtype: str = "bf16"

    @property
    def Wn(self) -> int:
        return len(self.parent)


@dataclass(frozen=True)
class LmHeadConfig:
    """LM head fused with E2E-TV: one trunk of L score rows plus R branches of
    Wn nodes (parent map as for the loss), hidden size H, vocabulary V.

    Value laws: draft and target hidden states N(0, 1) in bf16; both heads
    N(0, (sd / sqrt(H))^2) in bf16, independent, so every logit is about
    N(0, sd^2); anchors uniform without replacement in [P, L - 1); the target
    row of a node is its parent's branch row, or the anchor's trunk row for a
    node on the anchor (the score-row rule)."""

    L: int
    P: int
    R: int
    parent: Tuple[int, ...]
    H: int
    V: int
    sd: float = 2.0
    dtype: str = "bf16"
    T: int = 1

    @property
    def Wn(self) -> int:
        return len(self.parent)

    @property
    def B(self) -> int:
        return self.R


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    attn: Optional[AttnConfig]
    loss: Optional[LossConfig]
    gdn: Optional[GdnConfig] = None
    qsa: Optional[QsaConfig] = None
    lmhead: Optional[LmHeadConfig] = None


_C4P, _C4D = chain(4)
_C8P, _C8D = chain(8)
_C16P, _C16D = chain(16)
_C7P, _C7D = chain(7)

VOCAB = 151936

WORKLOADS = {
    1: Workload(
        1, "tiny",
        AttnConfig(T=1, L=64, P=16, B=4, parent=_C4P, depth=_C4D,
                   Hq=2, Hkv=1, D=64, dtype="f32"),
        LossConfig(R=4, parent=_C4P, V=1000, dtype="f32", recipe="indep", sd=2.0),
        qsa=QsaConfig(T=1, L=64, P=16, B=4, parent=_C4P, Di=64, topk=4),
    ),
    2: Workload(
        2, "layer8b",
        AttnConfig(T=1, L=4096, P=1024, B=64, parent=_C8P, depth=_C8D,
                   Hq=32, Hkv=8, D=128, dtype="bf16"),
        LossConfig(R=64, parent=_C8P, V=VOCAB, dtype="bf16", recipe="noise"),
        GdnConfig(T=1, L=4096, P=1024, B=64, parent=_C8P, H=32, D=128, dtype="bf16"),
        QsaConfig(T=1, L=4096, P=1024, B=64, parent=_C8P, Di=128, topk=64),
        LmHeadConfig(L=4096, P=1024, R=64, parent=_C8P, H=4096, V=VOCAB),
    ),
    3: Workload(
        3, "batch8",
        AttnConfig(T=8, L=8192, P=2048, B=128, parent=_C16P, depth=_C16D,
                   Hq=32, Hkv=8, D=128, dtype="bf16"),
        LossConfig(R=8 * 128, parent=_C16P, V=VOCAB, dtype="bf16",
                   recipe="rho", sd=3.0, rho=0.8),
        GdnConfig(T=8, L=8192, P=2048, B=128, parent=_C16P, H=32, D=128, dtype="bf16"),
        QsaConfig(T=8, L=8192, P=2048, B=128, parent=_C16P, Di=128, topk=512),
    ),
    4: Workload(
        4, "loss_stress",
        None,
        LossConfig(R=1024, parent=_C7P, V=VOCAB, dtype="bf16", recipe="stress"),
    ),
    5: Workload(
        5, "long",
        AttnConfig(T=1, L=32768, P=8192, B=512, parent=FORK_PARENT,
                   depth=FORK_DEPTH, Hq=24, Hkv=4, D=256, dtype="bf16"),
        LossConfig(R=512, parent=FORK_PARENT, V=VOCAB, dtype="bf16", recipe="noise"),
        GdnConfig(T=1, L=32768, P=8192, B=512, parent=FORK_PARENT, H=16, D=128, dtype="bf16"),
        QsaConfig(T=1, L=32768, P=8192, B=512, parent=FORK_PARENT, Di=128, topk=512),
    ),
}


def workload(cid: int) -> Workload:
    return WORKLOADS[cid]


def shrink_attn(cfg: AttnConfig, **kw) -> AttnConfig:
    """Same heads/dtype/tree, smaller trunk or fewer branches (parity sizes)."""
    return dataclasses.replace(cfg, **kw)


def shrink_loss(cfg: LossConfig, **kw) -> LossConfig:
    return dataclasses.replace(cfg, **kw)


def shrink_lmhead(cfg: LmHeadConfig, **kw) -> LmHeadConfig:
    return dataclasses.replace(cfg, **kw)


def shrink_qsa(cfg: QsaConfig, **kw) -> QsaConfig:
    return dataclasses.replace(cfg, **kw)


def shrink_gdn(cfg: GdnConfig, **kw) -> GdnConfig:
    return dataclasses.replace(cfg, **kw)
