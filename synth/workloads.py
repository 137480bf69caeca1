"""Layer shapes of the workloads.

Shapes come from the Qwen3.8-27B DFlash2 drafter model card (its property table:
hidden 5120, intermediate 17408, 32 query heads, 8 key/value heads, head
dimension 128, vocabulary 248320; and its quantised-layer table: the context
projection ``fc`` is 5120 x 25600 over five target layers).  Fused projections
concatenate output columns: q/k/v -> (32 + 2*8) * 128 = 6144, gate/up ->
2 * 17408 = 34816.
"""
from __future__ import annotations

from dataclasses import dataclass

HIDDEN = 5120
INTERMEDIATE = 17408
Q_HEADS = 32
KV_HEADS = 8
HEAD_DIM = 128
VOCAB = 248320
TARGET_LAYERS = 5
DRAFT_LAYERS = 5
GROUP = 128


@dataclass(frozen=True)
class Layer:
    name: str
    K: int
    N: int


QKV = Layer("qkv", HIDDEN, (Q_HEADS + 2 * KV_HEADS) * HEAD_DIM)
O_PROJ = Layer("o_proj", Q_HEADS * HEAD_DIM, HIDDEN)
GATE_UP = Layer("gate_up", HIDDEN, 2 * INTERMEDIATE)
DOWN = Layer("down", INTERMEDIATE, HIDDEN)
FC = Layer("fc", TARGET_LAYERS * HIDDEN, HIDDEN)
LM_HEAD = Layer("lm_head", HIDDEN, VOCAB)
SINGLE = Layer("single", 512, 256)

DECODE_LAYERS = (QKV, O_PROJ, GATE_UP, DOWN)
PREFILL_LAYERS = (QKV, O_PROJ, GATE_UP, DOWN, FC)

# One GPU's share under the tensor-parallel size 4 both serving recipes fix (Flint card,
# serving recipe; target model card, serving section): the column-parallel layers (qkv,
# gate/up, vocabulary head) keep K and take N/4 output columns; the row-parallel ones
# (o_proj, down) keep N and take K/4, on 128-wide group boundaries (8 and 34 groups).
TP = 4
QKV_TP = Layer("qkv_tp4", HIDDEN, (Q_HEADS + 2 * KV_HEADS) * HEAD_DIM // TP)
O_PROJ_TP = Layer("o_proj_tp4", Q_HEADS * HEAD_DIM // TP, HIDDEN)
GATE_UP_TP = Layer("gate_up_tp4", HIDDEN, 2 * INTERMEDIATE // TP)
DOWN_TP = Layer("down_tp4", INTERMEDIATE // TP, HIDDEN)
LM_HEAD_TP = Layer("lm_head_tp4", HIDDEN, VOCAB // TP)
SHARD_LAYERS = (QKV_TP, O_PROJ_TP, GATE_UP_TP, DOWN_TP)

LAYERS = {l.name: l for l in (QKV, O_PROJ, GATE_UP, DOWN, FC, LM_HEAD, SINGLE, QKV_TP, O_PROJ_TP, GATE_UP_TP,
                              DOWN_TP, LM_HEAD_TP)}


def config(name: str) -> dict:
    """The five workloads: shapes, token counts and activation recipe."""
    table = {
        # one draft block through a single small W8A8 G128 linear, seed 0, no outliers
        "single": dict(M=[8], layers=[SINGLE], outliers=False, kind="w8a8"),
        # decode: 8 sequences x block 8 = 64 tokens through the four drafter linears
        "decode": dict(M=[64], layers=list(DECODE_LAYERS), outliers=True, kind="w8a8"),
        # prefill: 2048-token sliding window x 2 sequences, plus the context projection
        "prefill": dict(M=[4096], layers=list(PREFILL_LAYERS), outliers=True, kind="w8a8"),
        # INT8 vocabulary head at decode
        "lm_head": dict(M=[64], layers=[LM_HEAD], outliers=False, kind="w8a8"),
        # 4-bit weight-only sibling on the decode shapes
        "w4a16": dict(M=[8, 64], layers=list(DECODE_LAYERS), outliers=True, kind="w4a16"),
    }
    return table[name]
