"""Named workload shapes (synthetic; the pages publish no weights).

* ``tiny``: one layer, H 256, 16 experts of intermediate 128, top-2 plus a
  shared expert of 128; 4-bit experts, dense bf16 router.
* ``a3b``: the 35B-A3B shape of the PureDrive model card ("Summary"): 40
  layers, H 2048, 256 experts of intermediate 512, top-8 plus a shared expert
  of 512; 6-bit routed experts, 8-bit shared expert and router. T = 1, or
  T in {2, 4, 8} for multi-row verify ("How it works": the target verifies
  several rows in one pass reading the weights once).
* ``a17b``: the 397B-A17B shape of the flash-moe news page ("Model
  architecture"): 60 layers, H 4096, 512 experts of intermediate 1024, top-10
  plus a shared expert of 1024; 4-bit experts and shared expert, 8-bit router.
* ``a17b_lowbit``: 15 layers of the same width, top-4 plus shared, 3-bit
  routed experts (10 codes per word), 8-bit shared expert and router, T = 32.
"""

from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Dict


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    inter: int
    top_k: int
    shared_inter: int
    router_bits: int
    expert_bits: int
    shared_bits: int
    n_layers: int
    T: int
    rms_eps: float = 1e-6

    def shape_kwargs(self) -> Dict[str, int]:
        d = asdict(self)
        for k in ("name", "n_layers", "T"):
            d.pop(k)
        return d


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 256, 16, 128, 2, 128, 16, 4, 4, n_layers=1, T=1),
    "a3b": Workload("a3b", 2048, 256, 512, 8, 512, 8, 6, 8, n_layers=40, T=1),
    "a3b_verify": Workload("a3b_verify", 2048, 256, 512, 8, 512, 8, 6, 8, n_layers=40, T=8),
    "a17b": Workload("a17b", 4096, 512, 1024, 10, 1024, 8, 4, 4, n_layers=60, T=1),
    "a17b_lowbit": Workload("a17b_lowbit", 4096, 512, 1024, 4, 1024, 8, 3, 8, n_layers=15, T=32),
}
