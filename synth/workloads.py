"""Matrix shapes, seeds and row counts of the workloads this library is measured on.

All shapes are (N outputs, K inputs).  One dense transformer layer of hidden
size 5120 with grouped-query attention (64 query heads, 8 key/value heads,
head_dim 128) and an MLP of width 25600; the full weight pass is 64 such layers
plus a 5120 -> 151936 output head.  Q|K|V share their input and so do gate|up;
the pass fuses each pair of siblings along N (one GEMM, y sliced afterwards).

Rows R stack the activations of several agents: each agent contributes its next
token plus two draft tokens, so 4 agents give R = 12 (OpenJet multi-agent serving
page, section on moving the weights only once).
"""
from __future__ import annotations

from dataclasses import dataclass

HIDDEN = 5120
Q_OUT = 8192        # 64 heads x 128
KV_OUT = 1024       # 8 heads x 128
MLP = 25600
VOCAB = 151936
LAYERS = 64

# matrix ids inside a layer (matrix id = layer * 8 + slot); the output head is 512
SLOT = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}
LM_HEAD_ID = 512

AGENTS = 4
ROWS_PER_AGENT = 3   # next token + 2 drafts
R_DEFAULT = AGENTS * ROWS_PER_AGENT


@dataclass(frozen=True)
class Mat:
    name: str
    N: int
    K: int
    mids: tuple          # matrix ids concatenated along N (fused siblings)
    splits: tuple        # N of each part, same order as mids

    @property
    def weights(self) -> int:
        return self.N * self.K

    @property
    def packed_bytes(self) -> int:
        return self.N * self.K // 256 * 144


def layer_mats(layer: int) -> list:
    """The four GEMMs of one layer, in dependency order, siblings fused."""
    b = layer * 8
    return [
        Mat("qkv", Q_OUT + 2 * KV_OUT, HIDDEN, (b + 0, b + 1, b + 2), (Q_OUT, KV_OUT, KV_OUT)),
        Mat("o", HIDDEN, Q_OUT, (b + 3,), (HIDDEN,)),
        Mat("gate_up", 2 * MLP, HIDDEN, (b + 4, b + 5), (MLP, MLP)),
        Mat("down", HIDDEN, MLP, (b + 6,), (HIDDEN,)),
    ]


def lm_head() -> Mat:
    return Mat("lm_head", VOCAB, HIDDEN, (LM_HEAD_ID,), (VOCAB,))


def full_pass() -> list:
    mats = []
    for layer in range(LAYERS):
        mats.extend(layer_mats(layer))
    mats.append(lm_head())
    return mats


def pass_bytes() -> int:
    return sum(m.packed_bytes for m in full_pass())


def pass_weights() -> int:
    return sum(m.weights for m in full_pass())


# the single-matrix correctness workload
SMALL = dict(N=256, K=1024, R=12, seed=0, mid=0)

# seeds per workload
SEED_SMALL, SEED_LAYER, SEED_PASS, SEED_RAGGED, SEED_LARGE_R = 0, 1, 2, 3, 4

# activation stream ids: one x per input width (no chaining between GEMMs)
X_STREAM = {HIDDEN: 1, Q_OUT: 2, MLP: 3}


def ragged_schedule(seed: int = SEED_RAGGED, steps: int = 100) -> list:
    """R_t = 3 * a_t with a_t ~ U{1..4} i.i.d. per step (seeded)."""
    from . import mix64
    out = []
    for t in range(steps):
        u = mix64(mix64(seed * 0x9E3779B97F4A7C15 + 0x5A17) ^ (t + 1))
        out.append(ROWS_PER_AGENT * (1 + (u >> 62)))
    return out
