"""The five synthetic workloads of the Ulysses attention share, and their inputs.

Shapes only: which tensors exist, their sizes and which random stream fills
them.  Stream numbers: 0 sample lengths, 1 Q (or fused QKV), 2 K (or fused
KV), 3 V, 4 dO, 5 per-token loss, 6 label ids.

Layouts (bf16 tensors are uint16 bit patterns):
  rank-share attention tensors  q, do: [N][hq][d]; k, v: [N][hkv][d]
  sequence-sharded exchange buffers  [P][N/P][G][H][d] (H = global head count)
  per-token loss / labels  [P][N/P]
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import gen

IGNORE_INDEX = -100
VOCAB = 128000


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    sp_size: int
    n_tokens: int
    hq: int              # query heads per rank (local)
    hkv: int             # KV heads per rank (local)
    head_dim: int
    pack: tuple | None = None        # (lo, hi) sample-length range, None = one sample
    prompt_frac: float = 0.0         # leading fraction of tokens labelled IGNORE_INDEX
    relayout_groups: int = 0         # G of the fused relayout-only workload (0: none)
    relayout_heads: int = 0          # global H of the relayout-only workload
    notes: str = field(default="", compare=False)

    @property
    def Hq(self) -> int:
        return self.hq * self.sp_size

    @property
    def Hkv(self) -> int:
        return self.hkv * self.sp_size

    def lengths(self) -> list[int]:
        if self.pack is None:
            return [self.n_tokens]
        return gen.sample_lengths((self.cfg, 0), self.n_tokens, *self.pack)

    def position_ids(self) -> np.ndarray:
        return gen.position_ids_from_lengths(self.lengths())

    def allowed_pairs(self) -> int:
        """Number of (query, key) pairs a causal, sample-bounded mask allows, per head."""
        return sum(L * (L + 1) // 2 for L in self.lengths())


WORKLOADS = {
    1: Workload(1, "tiny-full-layer-sp4-n1024", 4, 1024, 2, 2, 64,
                relayout_groups=3, relayout_heads=8,
                notes="all 4 rank buffers, QKV fused G=3, H=8"),
    2: Workload(2, "llama3-8b-share-sp4-n32768-packed", 4, 32768, 8, 2, 128, pack=(512, 8192)),
    3: Workload(3, "long-seq-share-sp8-n131072", 8, 131072, 4, 1, 128, prompt_frac=0.1),
    4: Workload(4, "relayout-p8-n262144-h32", 8, 262144, 0, 0, 128,
                relayout_groups=3, relayout_heads=32),
    5: Workload(5, "500k-share-sp8-n524288-packed", 8, 524288, 4, 1, 128,
                pack=(32768, 262144), prompt_frac=0.1),
}


def rank_share_inputs(w: Workload, with_grad: bool = True) -> dict:
    """q, k, v (and dO) drawn directly in the rank-share layout, plus position_ids."""
    N, d = w.n_tokens, w.head_dim
    out = {
        "q": gen.normal_bf16((w.cfg, 1), (N, w.hq, d)),
        "k": gen.normal_bf16((w.cfg, 2), (N, w.hkv, d)),
        "v": gen.normal_bf16((w.cfg, 3), (N, w.hkv, d)),
        "pos": w.position_ids(),
    }
    if with_grad:
        out["do"] = gen.normal_bf16((w.cfg, 4), (N, w.hq, d))
    return out


def exchange_inputs(w: Workload, with_grad: bool = True) -> dict:
    """Sequence-sharded exchange buffers for a workload whose step includes the relayout.

    GQA models exchange Q (G=1, H=Hq) and the fused K/V pair (G=2, H=Hkv)
    separately; when Hq == Hkv a single fused QKV buffer (G=3) is used."""
    P, N, d = w.sp_size, w.n_tokens, w.head_dim
    T = N // P
    out = {"pos": w.position_ids()}
    if w.Hq == w.Hkv:
        out["qkv_seq"] = gen.normal_bf16((w.cfg, 1), (P, T, 3, w.Hq, d))
    else:
        out["q_seq"] = gen.normal_bf16((w.cfg, 1), (P, T, 1, w.Hq, d))
        out["kv_seq"] = gen.normal_bf16((w.cfg, 2), (P, T, 2, w.Hkv, d))
    if with_grad:
        out["do_seq"] = gen.normal_bf16((w.cfg, 4), (P, T, 1, w.Hq, d))
    return out


def relayout_inputs(w: Workload) -> np.ndarray:
    """The fused buffer [P][N/P][G][H][d] of a relayout workload."""
    P, N = w.sp_size, w.n_tokens
    return gen.normal_bf16((w.cfg, 1), (P, N // P, w.relayout_groups, w.relayout_heads, w.head_dim))


def loss_inputs(w: Workload) -> dict:
    """Per-token loss ~ U[0, 12) and shift_labels with a prompt prefix of IGNORE_INDEX.

    The first round(prompt_frac * N) tokens of the (global) sequence are prompt;
    the rest carry label ids uniform in [0, VOCAB)."""
    P, N = w.sp_size, w.n_tokens
    token_loss = gen.uniform_f32((w.cfg, 5), (P, N // P), 0.0, 12.0)
    labels = gen.integers_i64((w.cfg, 6), (N,), 0, VOCAB)
    n_prompt = int(round(w.prompt_frac * N))
    labels[:n_prompt] = IGNORE_INDEX
    return {"token_loss": token_loss, "shift_labels": labels.reshape(P, N // P)}


# ---------------------------------------------------------------------------
# Per-token cross-entropy from hidden states (the loss ahead of the
# token-weighted aggregation): hidden states x ~ N(0,1), an LM-head matrix
# w ~ N(0, 1/hidden) (logits of order 1), labels uniform over the vocabulary
# with the first `prompt_frac` of the tokens ignored (a prompt prefix).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class LceWorkload:
    cfg: int
    name: str
    n_tokens: int
    hidden: int
    vocab: int
    prompt_frac: float = 0.1


LCE_WORKLOADS = {
    11: LceWorkload(11, "lce-small-n300-v1000-k256", 300, 256, 1000),
    12: LceWorkload(12, "lce-llama2-vocab-n1024-v32000-k1024", 1024, 1024, 32000),
    13: LceWorkload(13, "lce-llama3-8b-lmhead-n4096-v128256-k4096", 4096, 4096, 128256),
    14: LceWorkload(14, "lce-odd-vocab-n130-v997-k256", 130, 256, 997),
    15: LceWorkload(15, "lce-tiny-vocab-n70-v3-k512", 70, 512, 3),
}


def lce_inputs(w: LceWorkload) -> dict:
    """x [N][K] and w [V][K] bf16 bit patterns, labels [N] int64 (IGNORE_INDEX for
    the prompt prefix) and the token-weighted loss's upstream gradient g [N]
    (1/T on valid tokens)."""
    x = gen.normal_bf16((w.cfg, 1), (w.n_tokens, w.hidden))
    mat = gen.normal_bf16_scaled((w.cfg, 2), (w.vocab, w.hidden), 1.0 / w.hidden ** 0.5)
    labels = gen.integers_i64((w.cfg, 6), (w.n_tokens,), 0, w.vocab)
    n_prompt = int(round(w.prompt_frac * w.n_tokens))
    labels[:n_prompt] = IGNORE_INDEX
    T = int((labels != IGNORE_INDEX).sum())
    g = np.where(labels != IGNORE_INDEX, 1.0 / max(T, 1), 0.0).astype(np.float32)
    return {"x": x, "w": mat, "labels": labels, "g": g}
