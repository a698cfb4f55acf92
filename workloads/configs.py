"""The five decode workloads, as data.

Shapes follow the decode setting that the LeapQuant paper page ("LeapQuant:
Efficient Linear Attention with Accurate Recurrent State Quantization")
describes for Gated DeltaNet and Kimi Delta Attention layers: a 128x128 state
per (sequence, head, layer), a window of 16 tokens (the main configuration
named in the news write-up "LeapQuant trims the memory burden of
linear-attention models") and a few compensator rows.

Field meanings
  gate      "gdn" (one scalar decay per state and token) or "kda" (a decay per
            key channel).
  batch, heads, layers
            number of states n = batch * heads * layers; layers are separate
            state slabs stepped by separate launches.
  steps     decoded tokens per state.
  p, r      window length and compensator count.
  outliers  "rows4x20": four distinct rows of the initial state scaled by 20;
            "pct1": each row and each column of the initial state scaled, with
            probability 0.01, by a factor drawn from U(10, 30).
  snapshot_every
            tokens between prefix-cache snapshots (0: none).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    gate: str
    batch: int
    heads: int
    layers: int
    steps: int
    p: int
    r: int
    outliers: str
    dk: int = 128
    dv: int = 128
    snapshot_every: int = 0
    seed: int = 0

    @property
    def n_states(self) -> int:
        return self.batch * self.heads * self.layers

    @property
    def states_per_layer(self) -> int:
        return self.batch * self.heads

    @property
    def windows(self) -> int:
        return self.steps // self.p


_ALL = (
    WorkloadConfig("gdn_single_head_b1", "gdn", 1, 1, 1, 256, 16, 4, "rows4x20"),
    WorkloadConfig("gdn_layer_h32_b64", "gdn", 64, 32, 1, 4096, 16, 4, "pct1"),
    WorkloadConfig("gdn_b256_h32_4layers", "gdn", 256, 32, 4, 1024, 16, 4, "pct1"),
    WorkloadConfig("kda_h32_b128", "kda", 128, 32, 1, 2048, 16, 8, "pct1"),
    WorkloadConfig("gdn_long64k_h16_b8", "gdn", 8, 16, 1, 65536, 16, 4, "pct1", snapshot_every=1024),
)
WORKLOADS = {w.name: w for w in _ALL}
HEADLINE = "gdn_b256_h32_4layers"  # the throughput workload: batch 256 x 32 heads x 4 layers


def get_workload(name: str) -> WorkloadConfig:
    return WORKLOADS[name]
