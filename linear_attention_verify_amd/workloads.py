"""Seeded synthetic workloads for the GatedDeltaNet speculative verify/commit step.

This module only draws inputs. It holds none of the method's arithmetic, so both
the HIP path and the CPU oracle may consume what it produces. Everything is
numpy; bf16 tensors are carried as ``uint16`` bit patterns (round-to-nearest-even
from the fp32 draw) so that either side can decode them exactly.

Shapes follow the Qwen3-Next-style linear-attention layer the pages verify on
(LightLLM PR #1330 "Qwen3.5 / Qwen3.5-MoE MTP speculative decoding", Summary:
hybrid full-attention + Gated Delta Net models; FreeToken PR #844, Summary: k
defaults to 3 and goes up to 8). The pages print no activations, so every value
is synthetic:

    x [B][R][C]          N(0, 1)       pre-conv mixed q|k|v channels
    conv_w [C][W]        N(0, 1/W)
    alpha, beta [B][R][HV]  U(0.9, 1), U(0, 1)
    committed S, conv history of active slots  N(0, 1)
    inactive slots       NaN sentinels (fp32 0x7FC01234, bf16 0x7FC1)
    slot ids             distinct draw without replacement from the pool
    accept_len           U{1..R}, or geometric(p) capped at R
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32_SENTINEL = np.uint32(0x7FC01234)
BF16_SENTINEL = np.uint16(0x7FC1)


@dataclass(frozen=True)
class LayerShape:
    """One GatedDeltaNet layer as the verify/commit step sees it."""

    num_k_heads: int
    num_v_heads: int
    d_k: int
    d_v: int
    conv_width: int = 4
    dtype: str = "bf16"          # storage type of x, conv history, conv weights, gates, o
    act: str = "silu"            # activation after the causal conv: "silu" or "none"
    scale: float = 1.0           # o = scale * S q
    l2_eps: float = 1e-6         # q / sqrt(sum q^2 + eps)

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_k_heads * self.d_k + self.num_v_heads * self.d_v

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    batch: int
    rows: int
    num_slots: int
    layers: int = 1
    accept: str = "uniform"      # "uniform" -> U{1..rows}; "geometric" -> min(Geom(p), rows)
    accept_p: float = 0.3
    seed: int = 0
    modes: tuple = ("replay",)


QWEN3_NEXT_LAYER = LayerShape(num_k_heads=16, num_v_heads=32, d_k=128, d_v=128)

WORKLOADS = {
    "tiny-fp32": Workload(
        "tiny-fp32",
        LayerShape(num_k_heads=2, num_v_heads=4, d_k=32, d_v=32, dtype="f32"),
        batch=1, rows=3, num_slots=4, seed=0, modes=("replay", "snapshot")),
    "single-stream": Workload(
        "single-stream", QWEN3_NEXT_LAYER, batch=1, rows=3, num_slots=4, seed=1,
        modes=("replay", "snapshot")),
    "low-concurrency": Workload(
        "low-concurrency", QWEN3_NEXT_LAYER, batch=16, rows=4, num_slots=64, seed=2,
        modes=("replay", "snapshot")),
    "saturated-b64": Workload(
        "saturated-b64", QWEN3_NEXT_LAYER, batch=64, rows=9, num_slots=256,
        accept="geometric", accept_p=0.3, seed=3, modes=("replay", "snapshot")),
    "stack36": Workload(
        "stack36", QWEN3_NEXT_LAYER, batch=128, rows=4, num_slots=512, layers=36, seed=4,
        modes=("replay",)),
    # one rank's share of the layer under tensor parallelism over value heads
    # at TP4 (4 key / 8 value heads, C = 2048): the saturated batch's share, and
    # the batch at which a rank's share fills the chip as the saturated batch
    # fills it without sharding (1,024 units)
    "tp4-b64": Workload(
        "tp4-b64", LayerShape(num_k_heads=4, num_v_heads=8, d_k=128, d_v=128), batch=64, rows=9,
        num_slots=256, accept="geometric", accept_p=0.3, seed=5, modes=("replay", "snapshot")),
    "tp4-b256": Workload(
        "tp4-b256", LayerShape(num_k_heads=4, num_v_heads=8, d_k=128, d_v=128), batch=256, rows=9,
        num_slots=1024, accept="geometric", accept_p=0.3, seed=6, modes=("replay", "snapshot")),
}
WORKLOAD_ORDER = ["tiny-fp32", "single-stream", "low-concurrency", "saturated-b64", "stack36"]
TP_SHARES = ["tp4-b64", "tp4-b256"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); inputs here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return np.ascontiguousarray(a) if dtype == "f32" else f32_to_bf16_bits(a)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return np.asarray(a, dtype=np.float32) if dtype == "f32" else bf16_bits_to_f32(a)


def sentinel_fill(shape, dtype: str) -> np.ndarray:
    """An array of NaN sentinels in the given storage type ("f32", "bf16")."""
    if dtype == "f32":
        return np.full(shape, F32_SENTINEL, dtype=np.uint32).view(np.float32)
    return np.full(shape, BF16_SENTINEL, dtype=np.uint16)


def draw_requests(w: Workload, seed: int | None = None):
    """Per-request draws shared by every layer: slot ids and accept lengths."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    slot_ids = rng.choice(w.num_slots, size=w.batch, replace=False).astype(np.int32)
    if w.accept == "uniform":
        accept = rng.integers(1, w.rows + 1, size=w.batch)
    elif w.accept == "geometric":
        accept = np.minimum(rng.geometric(w.accept_p, size=w.batch), w.rows)
    else:
        raise ValueError(w.accept)
    return slot_ids, accept.astype(np.int32)


def draw_layer(w: Workload, layer: int = 0, seed: int | None = None):
    """Per-layer draws in storage types.

    Returns a dict with ``ssm_active`` [B][HV][d_k][d_v] fp32 (pool layout: the
    transpose of each head's d_v x d_k state, d_v contiguous), ``conv_active``
    [B][W-1][C], ``conv_w`` [C][W], ``x`` [B][R][C], ``alpha``/``beta`` [B][R][HV].
    Entry b of the *_active arrays is the committed state of request b's slot.
    """
    s = w.shape
    base = w.seed if seed is None else seed
    rng = np.random.default_rng([base, layer])
    B, R, C, W = w.batch, w.rows, s.conv_channels, s.conv_width
    HV = s.num_v_heads
    f32 = np.float32
    x = rng.standard_normal((B, R, C), dtype=f32)
    conv_w = (rng.standard_normal((C, W), dtype=f32) / np.sqrt(W)).astype(f32)
    alpha = rng.uniform(0.9, 1.0, size=(B, R, HV)).astype(f32)
    beta = rng.uniform(0.0, 1.0, size=(B, R, HV)).astype(f32)
    conv_active = rng.standard_normal((B, W - 1, C), dtype=f32)
    ssm_active = rng.standard_normal((B, HV, s.d_k, s.d_v), dtype=f32)
    return {
        "x": to_storage(x, s.dtype),
        "conv_w": to_storage(conv_w, s.dtype),
        "alpha": to_storage(alpha, s.dtype),
        "beta": to_storage(beta, s.dtype),
        "conv_active": to_storage(conv_active, s.dtype),
        "ssm_active": ssm_active,
    }


def build_pools(w: Workload, layer_draw: dict, slot_ids: np.ndarray):
    """Full host pools: sentinels everywhere, the drawn states at the active slots."""
    s = w.shape
    ssm = sentinel_fill((w.num_slots, s.num_v_heads, s.d_k, s.d_v), "f32")
    conv = sentinel_fill((w.num_slots, s.conv_width - 1, s.conv_channels), s.dtype)
    valid = (slot_ids >= 0) & (slot_ids < w.num_slots)
    ssm[slot_ids[valid]] = layer_draw["ssm_active"][valid]
    conv[slot_ids[valid]] = layer_draw["conv_active"][valid]
    return ssm, conv


def draw_tokens(w: Workload, accept: np.ndarray, vocab: int = 151936, seed: int | None = None):
    """Draft tokens [B][R-1] and target greedy tokens [B][R] (int32) under
    which greedy acceptance yields exactly ``accept`` (entries 0 are treated
    as 1: padding requests still get tokens): the first n-1 drafts equal the
    target's tokens before them, and draft n (if any) differs."""
    rng = np.random.default_rng([w.seed if seed is None else seed, 7919])
    B, R = w.batch, w.rows
    draft = rng.integers(0, vocab, size=(B, R - 1)).astype(np.int32)
    target = rng.integers(0, vocab, size=(B, R)).astype(np.int32)
    for b in range(B):
        n = max(int(accept[b]), 1)
        target[b, :n - 1] = draft[b, :n - 1]
        if n - 1 < R - 1 and target[b, n - 1] == draft[b, n - 1]:
            target[b, n - 1] = (draft[b, n - 1] + 1) % vocab
    return draft, target


def small_workload(shape: LayerShape, batch: int, rows: int, num_slots: int, seed: int,
                   name: str = "custom", **kw) -> Workload:
    return Workload(name=name, shape=shape, batch=batch, rows=rows, num_slots=num_slots,
                    seed=seed, **kw)


# ---- verification attention (the hybrid model's full-attention layers) ----

@dataclass(frozen=True)
class AttnShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 64
    scale: float | None = None    # None: 1 / sqrt(head_dim)

    def __post_init__(self):
        if self.scale is None:
            object.__setattr__(self, "scale", 1.0 / float(np.sqrt(self.head_dim)))


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    shape: AttnShape
    batch: int
    rows: int
    min_len: int          # seq_len drawn uniformly in [min_len, max_len] (verify rows included)
    max_len: int
    seed: int = 0
    padding: tuple = ()   # requests left as padding (seq_len 0)

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.shape.page_size)


ATTN_WORKLOADS = {
    # Qwen3-Next-like full-attention layer: 16 query / 2 KV heads of 256
    "attn-b64": AttnWorkload("attn-b64", AttnShape(16, 2, 256, 64), batch=64, rows=9,
                             min_len=1024, max_len=8192, seed=11),
    "attn-single": AttnWorkload("attn-single", AttnShape(16, 2, 256, 64), batch=1, rows=3,
                                min_len=2048, max_len=2048, seed=12),
}


def draw_attention(w: AttnWorkload):
    """seq_lens [B], block_table [B][max_blocks] (distinct pages per request, in
    random order, unused entries -1), and as bf16 bits: q [B][R][Hq][D] and the
    k/v caches [pages][page_size][Hkv][D], every value ~ N(0,1)."""
    s = w.shape
    rng = np.random.default_rng([w.seed, 31])
    B, R, D = w.batch, w.rows, s.head_dim
    seq = rng.integers(max(w.min_len, R), w.max_len + 1, size=B).astype(np.int32)
    for b in w.padding:
        seq[b] = 0
    mb = w.max_blocks
    need = -(-seq // s.page_size)
    pages = int(need.sum()) + 3
    perm = rng.permutation(pages).astype(np.int32)
    table = np.full((B, mb), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    f32 = np.float32
    q = to_storage(rng.standard_normal((B, R, s.num_q_heads, D), dtype=f32), "bf16")
    kc = to_storage(rng.standard_normal((pages, s.page_size, s.num_kv_heads, D), dtype=f32), "bf16")
    vc = to_storage(rng.standard_normal((pages, s.page_size, s.num_kv_heads, D), dtype=f32), "bf16")
    return {"seq_lens": seq, "block_table": table, "q": q, "k_cache": kc, "v_cache": vc}


# ---- speculative sampling of the verify rows' logits ----

@dataclass(frozen=True)
class SampleWorkload:
    name: str
    batch: int
    rows: int
    vocab: int
    draft_probs: bool = False     # a drafter that reports its distribution (else greedy)
    penalties: bool = True
    seed: int = 0
    boost: float = 15.0           # logit added to each row's likely token
    agree: float = 0.8            # chance that a draft is the previous row's likely token


SAMPLE_WORKLOADS = {
    # Qwen-sized vocabulary, the saturated batch's 64 requests x 9 rows
    "sample-b64": SampleWorkload("sample-b64", batch=64, rows=9, vocab=151936, seed=21),
}


def draw_sample(w: SampleWorkload):
    """Logits [B][R][V] ~ N(0, 4) rounded to bf16, with a likely token per row
    (logit + boost); drafts [B][R-1] equal to the previous row's likely token
    with probability `agree`, else uniform; temperatures U(0.7, 1.3);
    presence U(0, 1), frequency U(0, 0.5); prior counts mostly 0, else 1..3;
    pending tokens uniform. All int32 / fp32 numpy arrays, logits as bf16 bits."""
    rng = np.random.default_rng([w.seed, 97])
    B, R, V = w.batch, w.rows, w.vocab
    logits = 2.0 * rng.standard_normal((B, R, V), dtype=np.float32)
    likely = rng.integers(0, V, (B, R))
    np.put_along_axis(logits, likely[..., None], np.take_along_axis(logits, likely[..., None], 2) + w.boost, 2)
    draft = np.where(rng.random((B, R - 1)) < w.agree, likely[:, :R - 1], rng.integers(0, V, (B, R - 1)))
    d = {"logits": f32_to_bf16_bits(logits), "draft": draft.astype(np.int32),
         "temperature": rng.uniform(0.7, 1.3, B).astype(np.float32),
         "pending": rng.integers(0, V, B).astype(np.int32)}
    if w.penalties:
        d["presence"] = rng.uniform(0.0, 1.0, B).astype(np.float32)
        d["frequency"] = rng.uniform(0.0, 0.5, B).astype(np.float32)
        d["prior_counts"] = np.where(rng.random((B, V)) < 0.95, 0, rng.integers(1, 4, (B, V))).astype(np.int32)
    return d
