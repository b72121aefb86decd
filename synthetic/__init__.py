"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Holds sizes, value distributions and tree shapes only."""

from .configs import (AttnConfig, LossConfig, GdnConfig, Workload, WORKLOADS, workload,
                      shrink_attn, shrink_loss, shrink_gdn, shrink_qsa, QsaConfig, LmHeadConfig, shrink_lmhead, chain, FORK_PARENT, FORK_DEPTH, VOCAB)
from .gen import gen_attn, gen_loss, gen_prefill, gen_gdn, gen_gdn_conv, gen_qsa, gen_lmhead, anchors_for, stress_classes, derive_seed

__all__ = [
    "AttnConfig", "LossConfig", "GdnConfig", "shrink_gdn", "gen_gdn", "gen_gdn_conv", "Workload", "WORKLOADS", "workload", "shrink_attn",
    "shrink_loss", "chain", "FORK_PARENT", "FORK_DEPTH", "VOCAB", "gen_attn",
    "gen_loss", "gen_prefill", "anchors_for", "stress_classes", "derive_seed",
    "QsaConfig", "shrink_qsa", "gen_qsa", "LmHeadConfig", "shrink_lmhead", "gen_lmhead",
]
