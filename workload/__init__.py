"""Seeded synthetic inputs for the speculative-decoding verification step.

This module only draws random numbers and lays them out; it holds none of the
verification arithmetic (no norm, no matmul, no softmax, no sampling rule).
Both the CPU oracle and the GPU path consume exactly the arrays made here.

Workloads (shapes and distributions of the synthetic targets):

* ``tiny-fp32``             d=256, ffn=1024, L=2, V=4096, fp32 weights with
                            variance 1/d, B=1, K=4, sigma=0.5, T=1.
* ``8b-shaped-b1-k4``       d=4096, ffn=14336, L=8, V=32000, bf16 weights with
                            std 0.02, B=1, K=4, sigma=0.3, T=1.
* ``8b-shaped-sweep``       the same stack, B in {1,4,16,64} x K in {1,2,4,8}.
* ``70b-layer-share-b8-k4`` d=8192, ffn=28672, L=4, V=128256, bf16, B=8, K=4,
                            sigma=0.3, T=1 and T=0.
* ``large-batch-b256-k2``   d=4096, ffn=14336, L=8, V=128256, bf16, B=256,
                            K=2, sigma=0.5, T=0.7.

The draft model is an EAGLE-style head that reads the target's own final
hidden state (klu.ai glossary, "Variants: Draft Models, EAGLE, Medusa, and
Model-Free Methods"): its head weight is ``W_head + sigma * E`` with ``E``
distributed like ``W_head``, so sigma alone sets how far q is from p.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "SWEEP_B", "SWEEP_K", "SWEEP_SIGMA",
    "make_model", "make_hidden", "make_synthetic_logits", "make_random_tokens",
    "KV_BLOCK", "make_paged_attention", "ATTN_WORKLOADS",
    "MoEWorkload", "MOE_WORKLOADS", "make_moe_model", "make_embedding", "make_start_tokens",
    "bf16_bits_to_f32", "f32_to_bf16_bits",
]


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    ffn: int
    n_layers: int
    vocab: int
    wdtype: str          # "f32" or "bf16"
    B: int
    K: int
    sigma: float
    temperature: float
    init: str            # "var_inv_d" (variance 1/d) or "std_0.02"
    seed: int = 0

    @property
    def M(self) -> int:
        return self.B * (self.K + 1)

    @property
    def weight_std(self) -> float:
        return float(np.sqrt(1.0 / self.d)) if self.init == "var_inv_d" else 0.02

    def with_batch(self, B: int, K: int, **kw) -> "Workload":
        return replace(self, B=B, K=K, **kw)

    def weight_elems(self) -> int:
        return self.n_layers * 2 * self.d * self.ffn + self.vocab * self.d


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32", 256, 1024, 2, 4096, "f32", 1, 4, 0.5, 1.0, "var_inv_d"),
        Workload("8b-shaped-b1-k4", 4096, 14336, 8, 32000, "bf16", 1, 4, 0.3, 1.0, "std_0.02"),
        Workload("8b-shaped-sweep", 4096, 14336, 8, 32000, "bf16", 1, 1, 0.1, 1.0, "std_0.02"),
        Workload("70b-layer-share-b8-k4", 8192, 28672, 4, 128256, "bf16", 8, 4, 0.3, 1.0, "std_0.02"),
        Workload("large-batch-b256-k2", 4096, 14336, 8, 128256, "bf16", 256, 2, 0.5, 0.7, "std_0.02"),
    ]
}
SWEEP_B = (1, 4, 16, 64)
SWEEP_K = (1, 2, 4, 8)
SWEEP_SIGMA = (0.1, 0.5)

_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))

# Stream ids keep every tensor's draws independent of every other tensor's.
_STREAM = {"w_up": 1, "w_down": 2, "w_head": 3, "e_head": 4, "hidden": 5,
           "logits_t": 6, "logits_noise": 7, "tokens": 8, "kv": 9, "kv_table": 10,
           "moe_router": 11, "moe_up": 12, "moe_down": 13, "embed": 14, "start": 15}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest, ties to even);
    returns the 16-bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(shape, std: float, seed: int, stream: int, sub: int = 0) -> np.ndarray:
    """fp32 N(0, std^2) array; drawn in fixed chunks, each from its own
    PCG64 stream, so the result does not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunks = [(i, min(i + _CHUNK, n)) for i in range(0, n, _CHUNK)]

    def fill(ci):
        lo, hi = chunks[ci]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, sub, ci])))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if len(chunks) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(chunks))))
    return out.reshape(shape)


def _as_weight(x: np.ndarray, wdtype: str) -> np.ndarray:
    if wdtype == "f32":
        return x
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    n = flat_in.size

    def conv(lo):
        hi = min(lo + _CHUNK, n)
        flat_out[lo:hi] = f32_to_bf16_bits(flat_in[lo:hi])

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(conv, range(0, n, _CHUNK)))
    return out


def make_model(w: Workload, sigma: float | None = None, draft_head: bool = True) -> dict:
    """Target weights (row-major [out, in]) plus the draft head.

    Returns a dict with ``w_up`` [L, ffn, d], ``w_down`` [L, d, ffn],
    ``gain`` [L+1, d] fp32 (ones; the last row is the final norm),
    ``w_head`` [V, d] and, if asked, ``w_draft_head`` [V, d].  bf16 tensors
    are uint16 bit patterns; fp32 tensors are float32.
    """
    sigma = w.sigma if sigma is None else sigma
    std = w.weight_std
    L, d, f, V = w.n_layers, w.d, w.ffn, w.vocab
    model = {
        "w_up": _as_weight(_normal((L, f, d), std, w.seed, _STREAM["w_up"]), w.wdtype),
        "w_down": _as_weight(_normal((L, d, f), std, w.seed, _STREAM["w_down"]), w.wdtype),
        "gain": np.ones((L + 1, d), dtype=np.float32),
    }
    head32 = _normal((V, d), std, w.seed, _STREAM["w_head"])
    model["w_head"] = _as_weight(head32, w.wdtype)
    if draft_head:
        model["w_draft_head"] = make_draft_head(w, model["w_head"], sigma)
    return model


def make_draft_head(w: Workload, w_head: np.ndarray, sigma: float) -> np.ndarray:
    """Draft head W_head + sigma * E for the stored target head `w_head` (bf16
    bit patterns or fp32, after rounding), rounded to the weight dtype; E is
    drawn like W_head from its own stream, the same for every sigma."""
    base = w_head if w.wdtype == "f32" else bf16_bits_to_f32(w_head)
    e = _normal((w.vocab, w.d), w.weight_std, w.seed, _STREAM["e_head"])
    e *= np.float32(sigma)
    e += base
    return _as_weight(e, w.wdtype)


def make_hidden(w: Workload, M: int | None = None, sub: int = 0) -> np.ndarray:
    """Hidden-state inputs [M, d], fp32 N(0, 1)."""
    M = w.M if M is None else M
    return _normal((M, w.d), 1.0, w.seed, _STREAM["hidden"], sub)


def make_embedding(w: Workload) -> np.ndarray:
    """Token embedding table [V, d], fp32 N(0, 1): the input row of a
    position holding token x is row x (the same law as the hidden-state
    inputs of the verification workloads)."""
    return _normal((w.vocab, w.d), 1.0, w.seed, _STREAM["embed"])


def make_start_tokens(V: int, B: int, seed: int = 0, sub: int = 0) -> np.ndarray:
    """B starting tokens, uniform over [0, V), int32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _STREAM["start"], sub])))
    return g.integers(0, V, size=B, dtype=np.int32)


def make_synthetic_logits(B: int, K: int, V: int, scale: float, sigma: float,
                          seed: int = 0, sub: int = 0):
    """Logit-space stand-ins for the accept stage alone.

    target [B, K+1, V] ~ N(0, scale^2); draft [B, K, V] = target[:, :K] +
    sigma * scale * N(0, 1).  ``scale`` mimics the spread of a normed head's
    logits (about sqrt(d) * std(W_head)), ``sigma`` the draft head's offset.
    """
    t = _normal((B, K + 1, V), scale, seed, _STREAM["logits_t"], sub)
    n = _normal((B, K, V), sigma * scale, seed, _STREAM["logits_noise"], sub)
    n += t[:, :K, :]
    return t, n


def make_random_tokens(B: int, K: int, V: int, seed: int = 0, sub: int = 0) -> np.ndarray:
    """Uniform token ids [B, K] int32 (used where any valid draft will do)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _STREAM["tokens"], sub])))
    return g.integers(0, V, size=(B, K), dtype=np.int32)


# ---- paged KV cache for the attention of the verified positions -------------
KV_BLOCK = 32   # tokens per cache block

# Attention shapes of the targets above (grouped-query heads, head dim 128):
# Llama-8B-shaped 32 query / 8 KV heads, 70B-shaped 64 / 8, at the context
# lengths the co-design post measures attention at (32K and 128K are the
# post's; 4K and 8K are common serving contexts).
ATTN_WORKLOADS = {
    "8b-attn-b8-ctx8k": dict(B=8, Hq=32, Hkv=8, Dh=128, ctx=8192),
    "70b-attn-b8-ctx8k": dict(B=8, Hq=64, Hkv=8, Dh=128, ctx=8192),
    "8b-attn-b1-ctx32k": dict(B=1, Hq=32, Hkv=8, Dh=128, ctx=32768),
    "70b-attn-b4-ctx32k": dict(B=4, Hq=64, Hkv=8, Dh=128, ctx=32768),
    "8b-attn-b64-ctx4k": dict(B=64, Hq=32, Hkv=8, Dh=128, ctx=4096),
}


def make_paged_attention(B: int, T: int, Hq: int, Hkv: int, Dh: int, ctx, max_blocks: int,
                         spare_blocks: int = 3, seed: int = 0, sub: int = 0) -> dict:
    """A paged KV cache holding ctx[b] + T positions per request, in
    physically shuffled blocks, plus the step's queries and new keys/values.

    bf16 bit patterns (uint16) for q [B, T, Hq, Dh], k_new / v_new
    [B, T, Hkv, Dh], k_cache [nb, Hkv, KV_BLOCK, Dh], v_cache [nb, Hkv, Dh,
    KV_BLOCK]; block_table [B, max_blocks] int32 (unused entries 0), ctx_len
    [B] int32.  Values N(0, 1); the first ctx[b] positions are filled, the
    rest of the cache is left at zero for the step's append."""
    ctx = np.asarray(ctx, dtype=np.int32)
    need = [-(-(int(c) + T) // KV_BLOCK) for c in ctx]
    assert max(need) <= max_blocks, "max_blocks too small for ctx + T"
    nb = sum(need) + spare_blocks
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _STREAM["kv_table"], sub])))
    ids = g.permutation(nb).astype(np.int32)
    table = np.zeros((B, max_blocks), np.int32)
    o = 0
    for b in range(B):
        table[b, :need[b]] = ids[o:o + need[b]]
        o += need[b]

    def bf16(shape, stream_sub):
        return f32_to_bf16_bits(_normal(shape, 1.0, seed, _STREAM["kv"], sub * 16 + stream_sub))

    kc = np.zeros((nb, Hkv, KV_BLOCK, Dh), np.uint16)
    vc = np.zeros((nb, Hkv, Dh, KV_BLOCK), np.uint16)
    kfill, vfill = bf16((int(ctx.sum()) or 1, Hkv, Dh), 0), bf16((int(ctx.sum()) or 1, Hkv, Dh), 1)
    o = 0
    for b in range(B):
        for p in range(int(ctx[b])):
            blk, slot = table[b, p // KV_BLOCK], p % KV_BLOCK
            kc[blk, :, slot, :] = kfill[o]
            vc[blk, :, :, slot] = vfill[o]
            o += 1
    return {"q": bf16((B, T, Hq, Dh), 2), "k_new": bf16((B, T, Hkv, Dh), 3),
            "v_new": bf16((B, T, Hkv, Dh), 4), "k_cache": kc, "v_cache": vc,
            "block_table": table, "ctx_len": ctx.copy(), "num_blocks": nb}


# ---- mixture-of-experts target ------------------------------------------------
@dataclass(frozen=True)
class MoEWorkload:
    """A stack of pre-norm MoE blocks: a router [E, d] picks top_k of
    n_experts SiLU MLP experts (up [ffn, d], down [d, ffn]) per position; a
    final RMSNorm and the LM head follow.  bf16 weights, std 0.02."""
    name: str
    d: int
    ffn: int             # per expert
    n_experts: int
    top_k: int
    n_layers: int
    vocab: int
    B: int
    K: int
    sigma: float
    temperature: float
    seed: int = 0

    @property
    def M(self) -> int:
        return self.B * (self.K + 1)

    weight_std = 0.02

    def expert_elems(self) -> int:
        return 2 * self.d * self.ffn

    def with_batch(self, B: int, K: int, **kw) -> "MoEWorkload":
        return replace(self, B=B, K=K, **kw)


# 64 fine-grained experts, 6 active per position: a small-expert MoE whose
# expert weights (2.95 GB over 4 blocks) dominate, so the bytes a step streams
# grow with the number of distinct experts its B*(K+1) positions touch.
MOE_WORKLOADS = {
    "moe-64e-top6-b1-k4": MoEWorkload("moe-64e-top6-b1-k4", 2048, 1408, 64, 6, 4, 32000, 1, 4,
                                      0.3, 1.0),
}


def make_moe_model(w: MoEWorkload, sigma: float | None = None, draft_head: bool = True) -> dict:
    """MoE weights as bf16 bit patterns: ``w_router`` [L, E, d], ``w_up``
    [L, E, ffn, d], ``w_down`` [L, E, d, ffn], ``w_head`` [V, d] (and the
    draft head ``w_head + sigma E``), ``gain`` [L+1, d] ones."""
    sigma = w.sigma if sigma is None else sigma
    std = w.weight_std
    L, E, d, f, V = w.n_layers, w.n_experts, w.d, w.ffn, w.vocab
    model = {
        "w_router": _as_weight(_normal((L, E, d), std, w.seed, _STREAM["moe_router"]), "bf16"),
        "w_up": _as_weight(_normal((L, E, f, d), std, w.seed, _STREAM["moe_up"]), "bf16"),
        "w_down": _as_weight(_normal((L, E, d, f), std, w.seed, _STREAM["moe_down"]), "bf16"),
        "gain": np.ones((L + 1, d), dtype=np.float32),
    }
    head32 = _normal((V, d), std, w.seed, _STREAM["w_head"])
    model["w_head"] = _as_weight(head32, "bf16")
    if draft_head:
        e = _normal((V, d), std, w.seed, _STREAM["e_head"])
        e *= np.float32(sigma)
        e += bf16_bits_to_f32(model["w_head"])
        model["w_draft_head"] = _as_weight(e, "bf16")
    return model
