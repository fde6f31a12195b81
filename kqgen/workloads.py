"""The five synthetic workloads (shapes from muser-book Ch 13 sections 13.1
and 13.6: hidden 6,656; 32 heads x 128 = 4,096 and 2 KV heads x 128 = 256
outputs; 52 layers; and the 202,048-row LM-head scale of Ch 6 Figure 6.6),
and the rest of a layer's matvecs with the formats Ch 6 Figure 6.6 lists
for them (attention output, FFN gate/up/down, the Q5_K LM head, the draft
projections).

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
FFN_ROWS = 19968       # ffn_gate/up outputs = ffn_down inputs
DRAFT_ROWS = 1024      # draft k/v outputs
DRAFT_FC_COLS = 33280  # draft fc inputs


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


# The rest of a layer (Ch 6 Figure 6.6; Ch 13 section 13.6 puts o_proj at
# about 6 % and the FFN at about 82 % of a layer's projection bytes).  In a
# decode step each of these reads a different vector, so each is its own
# launch; gate and up read the same normed hidden and share one.
def attn_output(cfg: int = 6, layer: int = 0):
    # 4096 -> 6656, Q4_K
    return [[Tensor("attn_output", Q4_K, HIDDEN, Q_ROWS, (cfg, layer, 10), (cfg, layer, 110))]]


def ffn_gate_up(cfg: int = 6, layer: int = 0):
    # 6656 -> 19968 twice, Q4_K, one shared x
    x = (cfg, layer, 111)
    return [[Tensor("ffn_gate", Q4_K, FFN_ROWS, HIDDEN, (cfg, layer, 11), x),
             Tensor("ffn_up", Q4_K, FFN_ROWS, HIDDEN, (cfg, layer, 12), x)]]


def ffn_down(cfg: int = 6, layer: int = 0, fmt: int | None = None):
    # 19968 -> 6656; the release artifact alternates Q4_K / Q6_K by layer
    if fmt is None:
        fmt = Q6_K if layer % 2 else Q4_K
    return [[Tensor("ffn_down", fmt, HIDDEN, FFN_ROWS, (cfg, layer, 13), (cfg, layer, 113))]]


def layer_rest(cfg: int = 6, layer: int = 0):
    return attn_output(cfg, layer) + ffn_gate_up(cfg, layer) + ffn_down(cfg, layer)


def full_layer(cfg: int = 6, layer: int = 0):
    """A whole layer's projection matvecs in decode order: the Q/K/V/gate
    set, the attention output, the FFN gate/up pair and the FFN down."""
    qg = Q5_K if layer % 2 else Q4_K
    return [qkvg_layer(cfg, layer, qg)] + layer_rest(cfg, layer)


def lm_head_q5k(cfg: int = 7, rows: int = LM_ROWS):
    # the LM head as the release artifact ships it: Q5_K, 6656 -> 202,048
    return [[Tensor("lm_head_q5k", Q5_K, rows, HIDDEN, (cfg, 0, 0), (cfg, 0, 100))]]


def lm_head_q4k(cfg: int = 10, rows: int = LM_ROWS):
    # the same 6656 -> 202,048 shape in Q4_K (the embedding table's format),
    # for the traffic of the large-matrix path in each format
    return [[Tensor("lm_head_q4k", Q4_K, rows, HIDDEN, (cfg, 0, 0), (cfg, 0, 100))]]


def draft_projections(cfg: int = 8):
    """The draft model's k (Q4_K) and v (Q6_K), 6656 -> 1024 from one x, and
    its fc, 33280 -> 6656 Q4_K."""
    x = (cfg, 0, 100)
    return [[Tensor("draft_k", Q4_K, DRAFT_ROWS, HIDDEN, (cfg, 0, 0), x),
             Tensor("draft_v", Q6_K, DRAFT_ROWS, HIDDEN, (cfg, 0, 1), x)],
            [Tensor("draft_fc", Q4_K, HIDDEN, DRAFT_FC_COLS, (cfg, 0, 2), (cfg, 0, 101))]]


def embedding_table(cfg: int = 9, rows: int = LM_ROWS):
    """The token embedding table: 202,048 x 6656 Q4_K, the ~1.34 B
    parameters of Ch 13 section 13.6, the Q4_K table of Ch 6 section 6.5."""
    return Tensor("token_embd", Q4_K, rows, HIDDEN, (cfg, 0, 0), (cfg, 0, 100))


def total_weight_bytes(launches) -> int:
    return sum(t.weight_bytes for launch in launches for t in launch)
