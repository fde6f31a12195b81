"""The five synthetic workloads (shapes from muser-book Ch 13 sections 13.1
and 13.6: hidden 6,656; 32 heads x 128 = 4,096 and 2 KV heads x 128 = 256
outputs; 52 layers; and the 202,048-row LM-head scale of Ch 6 Figure 6.6).

Each workload is a list of "launches"; a launch is a list of tensors that
share one grid-split call.  A tensor is (name, fmt, rows, cols, seed key,
x key).  Tensors with the same x key read the same activation plane.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import Q4_K, Q5_K, Q6_K, BLOCK_BYTES

HIDDEN = 6656
Q_ROWS = 4096          # 32 heads x 128
KV_ROWS = 256          # 2 KV heads x 128
LAYERS = 52
LM_ROWS = 202048


@dataclass(frozen=True)
class Tensor:
    name: str
    fmt: int
    rows: int
    cols: int
    wkey: tuple
    xkey: tuple

    @property
    def weight_bytes(self) -> int:
        return self.rows * (self.cols // 256) * BLOCK_BYTES[self.fmt]


def single_q4k(cfg: int = 1):
    return [[Tensor("w", Q4_K, 256, HIDDEN, (cfg, 0, 0), (cfg, 0, 100))]]


def qkvg_layer(cfg: int, layer: int, qg_fmt: int = Q4_K):
    x = (cfg, layer, 100)
    return [Tensor("q", qg_fmt, Q_ROWS, HIDDEN, (cfg, layer, 0), x),
            Tensor("k", Q6_K, KV_ROWS, HIDDEN, (cfg, layer, 1), x),
            Tensor("v", Q6_K, KV_ROWS, HIDDEN, (cfg, layer, 2), x),
            Tensor("gate", qg_fmt, Q_ROWS, HIDDEN, (cfg, layer, 3), x)]


def qkvg_set(cfg: int = 2):
    return [qkvg_layer(cfg, 0)]


def qkvg_stream(cfg: int = 3, layers: int = LAYERS):
    # odd layers carry Q and gate as Q5_K, even layers as Q4_K
    return [qkvg_layer(cfg, i, Q5_K if i % 2 else Q4_K) for i in range(layers)]


def lm_head(cfg: int = 4, rows: int = LM_ROWS):
    return [[Tensor("lm_head", Q6_K, rows, HIDDEN, (cfg, 0, 0), (cfg, 0, 100))]]


def kv_pair(cfg: int = 5, swapped: bool = False):
    fk, fv = (Q5_K, Q6_K) if swapped else (Q6_K, Q5_K)
    s = 1 if swapped else 0
    return [[Tensor("k", fk, KV_ROWS, HIDDEN, (cfg, s, 1), (cfg, s, 101)),
             Tensor("v", fv, KV_ROWS, HIDDEN, (cfg, s, 2), (cfg, s, 102))]]


def total_weight_bytes(launches) -> int:
    return sum(t.weight_bytes for launch in launches for t in launch)
