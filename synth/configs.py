"""The five seeded synthetic workloads of the MoE layer (shapes, routing recipe).

Shapes follow the pages' models: a 48-layer, 512-expert, top-10 model
([Strata] "显存里缓存的是什么？"), and a 43-layer, 256-expert, top-6 model with
hidden 4096 ([FreeToken] 2.1-2.2), plus a tiny layer that the CPU oracle
finishes in seconds.  Activations are bf16 ~N(0,1); router, shared gate and
expert weights ~N(0, 0.02) (expert weights then block-FP4 quantised); seed 0.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    T: int          # tokens per call (per layer)
    H: int          # hidden
    I: int          # expert intermediate (routed and shared)
    E: int          # routed experts
    k: int          # top-k
    L: int          # layers
    router: str     # "matrix": logits = x @ W_r ; "zipf": logits drawn (Zipf popularity + Gumbel)
    steps: int = 1  # decode steps (C3: 64)
    zipf_s: float = 0.0
    epoch_len: int = 0  # steps per hot-set epoch (0: one epoch)
    staged: bool = False  # expert blobs start in pinned host memory (two-slot ring)
    cache_frac: float = 0.0  # > 0: blobs in pinned host memory, a device LRU cache of this share of them
    fmt: str = "nvfp4"  # expert blob format: "nvfp4" (E4M3 scale per 16, fp32 global) or "mx" (MXFP4)
    seed: int = 0

    @property
    def E1(self) -> int:
        return self.E + 1

    def epoch(self, step: int) -> int:
        return step // self.epoch_len if self.epoch_len else 0

    def dims(self) -> dict:
        return dict(T=self.T, H=self.H, I=self.I, E=self.E, k=self.k, L=self.L)


CONFIGS = {
    1: Config(1, "tiny", T=8, H=512, I=256, E=32, k=4, L=1, router="matrix"),
    2: Config(2, "decode48", T=4, H=2048, I=512, E=512, k=10, L=48, router="zipf", zipf_s=1.0),
    3: Config(3, "decode43x64", T=16, H=4096, I=2048, E=256, k=6, L=43, router="zipf", steps=64,
              zipf_s=1.2, epoch_len=16),
    4: Config(4, "prefill8192", T=8192, H=2048, I=512, E=512, k=10, L=1, router="matrix"),
    5: Config(5, "streamed4x4096", T=4096, H=4096, I=2048, E=256, k=6, L=4, router="zipf", zipf_s=1.2,
              staged=True),
    # partial residency: decode48's shapes, a hot set that moves every 16 of 64
    # steps, and a device cache of one eighth of the (layer, expert) blobs
    6: Config(6, "cached48x64", T=4, H=2048, I=512, E=512, k=10, L=48, router="zipf", steps=64, zipf_s=1.0,
              epoch_len=16, cache_frac=0.125),
    # prefill8192's shapes with natively MXFP4 experts ([FreeToken] 2.1): the
    # scaled-MFMA path (MXFP8 activations)
    7: Config(7, "prefill8192_mx", T=8192, H=2048, I=512, E=512, k=10, L=1, router="matrix", fmt="mx"),
    # decode48 with MXFP4 experts: the weight-streaming kernel on MX blobs
    8: Config(8, "decode48_mx", T=4, H=2048, I=512, E=512, k=10, L=48, router="zipf", zipf_s=1.0, fmt="mx"),
}


def config_by_name(name: str) -> Config:
    for c in CONFIGS.values():
        if c.name == name or str(c.cfg_id) == str(name):
            return c
    raise KeyError(name)
