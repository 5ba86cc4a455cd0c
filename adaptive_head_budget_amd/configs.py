"""The five synthetic workload shapes this library is sized and tested for.

Shapes only: no arithmetic of the method lives here.  Each entry names the
model family whose attention geometry it copies (query heads, KV heads, head
dimension) and the eviction setting it exercises.

Sources for the settings (page title, section):
  * Ada-KV notes, "实验环境 / 参数设置": window 32, max-pool kernel 7,
    safeguard alpha 0.2; eviction after each layer's prefill.
  * Ada-KV (arXiv 2407.11550 HTML), Section 4 "Datasets": Ruler at 16K; budgets
    as 20/40/60/80 % of the full cache; fixed budget 1024 per head.
  * LAVa notes, "实验环境": max-pool kernel 7 on every score vector; budgets
    written as multiples of H*L; 128K contexts in the latency study.
  * CriticalKV notes, "主实验": 40 % budget, Qwen2.5-32B among the models;
    "损失函数 / 训练策略": stage split alpha 0.5.
  * LaProx page, abstract and Section 3: Mistral-7B-Instruct (v0.3) is the
    model analysed; 5 % of the KV cache kept; one model-wide selection across
    heads and layers.  The window length is not given there; the other pages'
    32 is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple, Union


@dataclass(frozen=True)
class Workload:
    name: str
    hq: int                 # query heads
    hkv: int                # KV heads (GQA groups)
    d: int                  # head dimension
    n: int                  # cached tokens per head, window included
    w: int                  # observation window (last w tokens)
    pool: int               # max-pool kernel (odd; 1 = off)
    layers: int
    batch: int
    dtype: str              # "bf16" or "f32"
    scorer: str             # "snapkv", "lava", "criticalkv" or "laprox"
    budget: int             # snapkv/criticalkv: per instance, window included;
                            # lava, laprox: total over all layers, windows included
    alpha: Tuple[int, int] = (1, 5)   # Ada-KV safeguard as an exact rational
    ck: Tuple[int, int] = (1, 2)      # CriticalKV stage-1 share
    hidden: int = 0                   # CriticalKV, LaProx: model hidden size D
    eps: float = 1e-6                 # CriticalKV: additive epsilon
    sinks: int = 0                    # leading keys aligned with the queries
    tau: Union[Tuple[float, ...], Tuple[str, float, float]] = ("loguniform", 0.1, 3.0)
    reserve: int = 0                  # empty rows kept per head for appends
    decode_steps: int = 0             # decode queries run after eviction
    append: bool = True               # decode steps append one token per head
    alloc: str = ""                   # allocation mode; "" = the scorer's own
                                      # ("ada", "lava", "criticalkv", "global",
                                      # "floor", "streaming")
    stream_sinks: int = 4             # StreamingLLM: sink tokens kept per head

    @property
    def instances(self) -> int:
        return self.layers * self.batch

    @property
    def p(self) -> int:
        return self.n - self.w

    @property
    def group(self) -> int:
        return self.hq // self.hkv


TINY_MHA = Workload(
    name="tiny_mha_h4_d16_n64", hq=4, hkv=4, d=16, n=64, w=4, pool=3,
    layers=1, batch=1, dtype="f32", scorer="snapkv", budget=64,
    tau=(0.2, 0.5, 1.0, 3.0), sinks=0, reserve=0, decode_steps=1, append=False)

LLAMA8B_LAYER = Workload(
    name="llama3.1-8b_layer_n16384", hq=32, hkv=8, d=128, n=16384, w=32, pool=7,
    layers=1, batch=1, dtype="bf16", scorer="snapkv",
    budget=(20 * 8 * 16384) // 100, sinks=4, reserve=1, decode_steps=1)

LLAMA8B_MODEL = Workload(
    name="llama3.1-8b_32L_b4_n32768", hq=32, hkv=8, d=128, n=32768, w=32, pool=7,
    layers=32, batch=4, dtype="bf16", scorer="snapkv", budget=1024 * 8,
    sinks=4, reserve=128, decode_steps=128)

MISTRAL7B_LAVA = Workload(
    name="mistral-7b_lava_32L_n131072", hq=32, hkv=8, d=128, n=131072, w=32, pool=7,
    layers=32, batch=1, dtype="bf16", scorer="lava", budget=128 * 8 * 32,
    sinks=4, reserve=0, decode_steps=0)

QWEN32B_CK = Workload(
    name="qwen2.5-32b_criticalkv_n65536", hq=40, hkv=8, d=128, n=65536, w=32, pool=7,
    layers=1, batch=1, dtype="bf16", scorer="criticalkv",
    budget=(40 * 8 * 65536) // 100, hidden=5120, sinks=4, reserve=0, decode_steps=0)

MISTRAL7B_LAPROX = Workload(
    name="mistral-7b_laprox_32L_n32768", hq=32, hkv=8, d=128, n=32768, w=32, pool=1,
    layers=32, batch=1, dtype="bf16", scorer="laprox",
    budget=(5 * 32 * 8 * 32768) // 100, hidden=4096, sinks=4, reserve=0, decode_steps=0)

ALL = (TINY_MHA, LLAMA8B_LAYER, LLAMA8B_MODEL, MISTRAL7B_LAVA, QWEN32B_CK, MISTRAL7B_LAPROX)
BY_NAME = {c.name: c for c in ALL}


def scaled(cfg: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    from dataclasses import replace
    return replace(cfg, **changes)
