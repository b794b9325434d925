"""Seeded synthetic workloads for sink-aware GQA attention.

This module only draws numbers: document lengths and random tensors.  It holds
none of the method's arithmetic, and both the fp64 oracle and the HIP path
consume exactly the bits it produces.

Recipe (the same for every configuration):
  * document lengths from numpy ``default_rng(seed)``;
  * tensor values from one CPU ``torch.Generator`` seeded with ``seed``, drawn
    in float32 in the order q, k, v, sinks, qnorm_w, knorm_w, then rounded
    once (round-to-nearest-even) to the storage dtype;
  * Q/K/V ~ N(0, 1); sinks ~ N(sink_mean, 1) fp32; RMSNorm weights
    1 + N(0, 0.02) fp32 with one weight vector of head_dim entries per
    projection;
  * for the backward, the output gradient dout ~ N(0, 1) [T, Hq, d] from a
    second generator seeded with seed + 1, rounded to the storage dtype;
  * padded batches (pad_to > 0): every document sits at the start of a slot
    of pad_to rows (a BSHD batch [D, pad_to] viewed as THD) and the padding
    rows hold draws from the same generator like any other row.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple
    num_q_heads: int = 32
    num_kv_heads: int = 4
    head_dim: int = 128
    dtype: str = "bf16"          # storage dtype of q, k, v and out
    window: int = -1             # > 0: keys i-W < j <= i; < 0: causal
    use_rope: bool = False
    sink_mean: float = 0.0
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    pad_to: int = 0              # > 0: every document padded to a slot of pad_to rows
    description: str = field(default="", compare=False)

    @property
    def total_tokens(self) -> int:
        """Real tokens (padding excluded)."""
        return int(sum(self.lengths))

    @property
    def num_rows(self) -> int:
        """Rows of the q/k/v tensors: real tokens, or D * pad_to when padded."""
        return self.num_docs * self.pad_to if self.pad_to else self.total_tokens

    @property
    def num_docs(self) -> int:
        return len(self.lengths)


def _sliding_lengths(seed: int = 0):
    # 8 documents, integer lengths uniform over [256, 4096] inclusive
    return tuple(int(x) for x in np.random.default_rng(seed).integers(256, 4097, size=8))


def _mixed_lengths(seed: int = 0):
    # 512 documents, geometric lengths with mean 200 (p = 1/200, support >= 1),
    # clipped to [1, 2048]
    g = np.random.default_rng(seed).geometric(1.0 / 200.0, size=512)
    return tuple(int(x) for x in np.clip(g, 1, 2048))


def named_workloads(seed: int = 0) -> dict:
    """The five configurations (Mixed appears once per alternating call)."""
    mixed = _mixed_lengths(seed)
    return {
        "tiny": Workload("tiny", (128,), 4, 1, 64, "f32", -1, False, 0.0,
                         description="1 doc S=128, 4q/1kv, d=64, fp32, causal, no RoPE"),
        "sliding": Workload("sliding", _sliding_lengths(seed), window=1024, use_rope=True,
                            description="8 docs U[256,4096], W=1024, NeoX RoPE"),
        "full": Workload("full", (32768,), window=-1, use_rope=False,
                         description="1 doc S=32768, causal, no RoPE"),
        "long": Workload("long", (65536, 65536), window=4096, use_rope=True, sink_mean=2.0,
                         description="2 docs S=65536, W=4096, NeoX RoPE, sinks N(2,1)"),
        "mixed_sliding": Workload("mixed_sliding", mixed, window=512, use_rope=True,
                                  description="512 docs geometric mean 200 clip [1,2048], W=512 + RoPE"),
        "mixed_causal": Workload("mixed_causal", mixed, window=-1, use_rope=False,
                                 description="512 docs geometric mean 200 clip [1,2048], causal, no RoPE"),
        "sliding_bshd": Workload("sliding_bshd", _sliding_lengths(seed), window=1024,
                                 use_rope=True, pad_to=4096,
                                 description="BSHD batch 8 x 4096 with trailing padding, real "
                                             "lengths U[256,4096], W=1024, NeoX RoPE"),
    }


_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}


def cu_seqlens(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """CPU tensors for workload ``w``: q [T,Hq,d], k/v [T,Hkv,d] in w.dtype,
    cu_seqlens int32 [D+1], sinks fp32 [Hq], qnorm_w / knorm_w fp32 [d]; T is
    w.num_rows.  Padded workloads add cu_seqlens_padded int32 [D+1] (slot
    starts) and attention_mask bool [D, pad_to]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    T, Hq, Hkv, d = w.num_rows, w.num_q_heads, w.num_kv_heads, w.head_dim
    dt = _TORCH_DTYPES[w.dtype]
    q = torch.randn((T, Hq, d), generator=gen, dtype=torch.float32).to(dt)
    k = torch.randn((T, Hkv, d), generator=gen, dtype=torch.float32).to(dt)
    v = torch.randn((T, Hkv, d), generator=gen, dtype=torch.float32).to(dt)
    sinks = torch.randn((Hq,), generator=gen, dtype=torch.float32) + float(w.sink_mean)
    qnorm_w = 1.0 + 0.02 * torch.randn((d,), generator=gen, dtype=torch.float32)
    knorm_w = 1.0 + 0.02 * torch.randn((d,), generator=gen, dtype=torch.float32)
    out = {
        "q": q, "k": k, "v": v,
        "cu_seqlens": torch.from_numpy(cu_seqlens(w.lengths)),
        "sinks": sinks, "qnorm_w": qnorm_w, "knorm_w": knorm_w,
    }
    if w.pad_to:
        _, cp = padded_boundaries(w.lengths, [w.pad_to] * w.num_docs)
        out["cu_seqlens_padded"] = torch.from_numpy(cp)
        out["attention_mask"] = (torch.arange(w.pad_to)[None, :]
                                 < torch.tensor(w.lengths)[:, None])
    return out


def make_grad_output(w: Workload, seed: int = 0) -> torch.Tensor:
    """dout [T, Hq, d] in w.dtype for the backward of workload ``w``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed + 1)
    return torch.randn((w.num_rows, w.num_q_heads, w.head_dim), generator=gen,
                       dtype=torch.float32).to(_TORCH_DTYPES[w.dtype])


def custom_workload(lengths, num_q_heads=32, num_kv_heads=4, head_dim=128,
                    dtype="bf16", window=-1, use_rope=False, sink_mean=0.0,
                    name="custom") -> Workload:
    return Workload(name, tuple(int(x) for x in lengths), num_q_heads, num_kv_heads,
                    head_dim, dtype, int(window), bool(use_rope), float(sink_mean))


def sample_rows(lengths, window: int, n_random: int, seed: int = 0,
                edge: int = 64) -> np.ndarray:
    """Deterministic subset of query tokens for checks at sizes where every row
    is too costly for the oracle: each document's first and last ``edge``
    tokens, the tokens around the window edge, and ``n_random`` seeded tokens."""
    cu = cu_seqlens(lengths)
    picks = set()
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        picks.update(range(a, min(b, a + edge)))
        picks.update(range(max(a, b - edge), b))
        if window > 0:
            picks.update(range(a + max(0, window - 2), min(b, a + window + 2)))
    T = int(cu[-1])
    if T and n_random:
        rng = np.random.default_rng(seed + 12345)
        picks.update(int(x) for x in rng.integers(0, T, size=n_random))
    return np.array(sorted(picks), dtype=np.int32)


def padded_boundaries(lengths, slots):
    """cu_seqlens (prefix sums of the real lengths) and cu_seqlens_padded
    (prefix sums of the slot sizes) of a padded-THD batch: document n's real
    tokens open its slot of slots[n] tokens, padding fills the rest."""
    lengths = np.asarray(lengths, dtype=np.int64)
    slots = np.asarray(slots, dtype=np.int64)
    if np.any(lengths > slots):
        raise ValueError("a document is longer than its slot")
    return cu_seqlens(lengths), cu_seqlens(slots)
