"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Holds sizes, value distributions and tree shapes only."""

from .configs import (AttnConfig, LossConfig, Workload, WORKLOADS, workload,
                      shrink_attn, shrink_loss, chain, FORK_PARENT, FORK_DEPTH, VOCAB)
from .gen import gen_attn, gen_loss, gen_prefill, anchors_for, stress_classes, derive_seed

__all__ = [
    "AttnConfig", "LossConfig", "Workload", "WORKLOADS", "workload", "shrink_attn",
    "shrink_loss", "chain", "FORK_PARENT", "FORK_DEPTH", "VOCAB", "gen_attn",
    "gen_loss", "gen_prefill", "anchors_for", "stress_classes", "derive_seed",
]
