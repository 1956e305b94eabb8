"""Oracle target forward over all B*(K+1) verification positions (fp64).

What the pages fix: the target scores every drafted position in a single
forward pass that reads its weights once (onlylabs/Cohere "Hardware Aware
Dynamic Speculative Decoding", section "Hardware-aware dynamic SD": the
target processes BS x (K+1) tokens; publishertech, section 1 "The
Speculative Cycle").  The pages define no architecture; the synthetic target
is the plain reading of "RMSNorm -> up -> SiLU -> down -> LM head": a stack of
pre-norm residual MLP blocks without gate or bias, then a final RMSNorm and
the LM head.  Rows never interact (there is no attention), so every row is
computed independently.

Numerics: fp64 throughout, except that the matmul inputs -- the normed
activations a, the SiLU output s and the final normed activation a_f -- are
rounded to bf16 (round to nearest even) when the weights are bf16, because
the product is defined as bf16 inputs with fp32-or-better accumulation.  With
fp32 weights nothing is rounded.

``accum="f32"`` evaluates the same contract in fp32 wherever the contract
allows fp32 -- matmuls (BLAS sgemm), the residual stream, the RMSNorm and the
SiLU -- with the same bf16 rounding points.  It exists only to measure how
far two valid evaluations of this contract drift apart through the stack
(each bf16 rounding decision can flip when the pre-rounding value moves by
one fp32 rounding, and a random MLP stack amplifies the flips layer by
layer); comparisons against the GPU use the fp64 default.  ``k_order``
(fp32 only) picks one of many equally valid summation orders: order 0 sums
the reduction index in storage order, order n > 0 in a seeded permutation of
it (the same permutation on both operands, so only the rounding sequence
changes).

Pinned by: torch.nn.functional (rms_norm, silu, linear) in float64 composed
in the same block order; special cases (zero down weights leave h unchanged;
zero layers reduce to the head on norm(hidden)); RMSNorm's scale invariance;
bf16 rounding against torch's float32 -> bfloat16 conversion.
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-5
_HEAD_ROWS = 8192


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (8 significant bits,
    ties to even).  x = m * 2^e with 0.5 <= |m| < 1; keep round(m * 2^8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # np.rint: ties to even


def weights_f64(w: np.ndarray, lo: int | None = None, hi: int | None = None,
                dtype=np.float64) -> np.ndarray:
    """Rows [lo, hi) of a stored weight matrix as fp64 (bf16 patterns are
    uint16; fp32 matrices pass through).  The upcast is exact."""
    part = w[lo:hi]
    if part.dtype == np.uint16:
        return (part.astype(np.uint32) << 16).view(np.float32).astype(dtype)
    return part.astype(dtype)


def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * g, per row."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * g


def silu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u) = u / (1 + exp(-u))."""
    return u / (1.0 + np.exp(-u))


_ACCUM = {"f64": np.float64, "f32": np.float32}


def _perm(k_order: int, K: int, *tag) -> np.ndarray | None:
    """The seeded reduction-index permutation of order k_order (None: storage order)."""
    if not k_order:
        return None
    return np.random.default_rng((k_order, *tag)).permutation(K)


def _mm(a: np.ndarray, w: np.ndarray, perm) -> np.ndarray:
    """a . w^T, summing the shared index in the order perm (None: as stored)."""
    if perm is None:
        return a @ w.T
    return a[:, perm] @ w[:, perm].T


def head(a_f: np.ndarray, w_head: np.ndarray, accum: str = "f64", k_order: int = 0) -> np.ndarray:
    """Logits a_f . W_head^T, taking the head in row blocks to bound memory."""
    dt = _ACCUM[accum]
    V = w_head.shape[0]
    out = np.empty((a_f.shape[0], V), dtype=np.float64)
    a = a_f.astype(dt)
    perm = _perm(k_order, a.shape[1], 0x4EAD)
    for lo in range(0, V, _HEAD_ROWS):
        hi = min(lo + _HEAD_ROWS, V)
        out[:, lo:hi] = _mm(a, weights_f64(w_head, lo, hi, dt), perm)
    return out


def final_activation(model: dict, hidden: np.ndarray, eps: float = RMS_EPS,
                     accum: str = "f64", k_order: int = 0) -> np.ndarray:
    """Run the L blocks and the final norm; returns a_f [rows, d] (fp64 values;
    with accum="f32" every step is evaluated in fp32)."""
    dt = _ACCUM[accum]
    rnd = bf16_round if model["w_up"].dtype == np.uint16 else (lambda v: v)

    def rnd_dt(v):
        return rnd(np.asarray(v, dtype=np.float64)).astype(dt)

    h = np.asarray(hidden, dtype=dt)
    g = np.asarray(model["gain"], dtype=dt)
    L, ffn, d = model["w_up"].shape
    for l in range(L):
        a = rnd_dt(rmsnorm(h, g[l], dt(eps)))
        u = _mm(a, weights_f64(model["w_up"][l], dtype=dt), _perm(k_order, d, l, 0))
        s = rnd_dt(silu(u))
        h = h + _mm(s, weights_f64(model["w_down"][l], dtype=dt), _perm(k_order, ffn, l, 1))
    return rnd(np.asarray(rmsnorm(h, g[L], dt(eps)), dtype=np.float64))


def forward(model: dict, hidden: np.ndarray, heads=("w_head",), eps: float = RMS_EPS,
            accum: str = "f64", k_order: int = 0):
    """Logits [rows, V] (fp64) for each requested head of ``model``.
    Returns one array, or a tuple when several heads are asked for."""
    if k_order and accum != "f32":
        raise ValueError("k_order selects an fp32 summation order")
    a_f = final_activation(model, hidden, eps, accum, k_order)
    outs = tuple(head(a_f, model[name], accum, k_order) for name in heads)
    return outs[0] if len(outs) == 1 else outs


def truncated(model: dict, n_layers: int) -> dict:
    """The first n_layers blocks of ``model`` with its final norm and heads."""
    out = dict(model)
    out["w_up"] = model["w_up"][:n_layers]
    out["w_down"] = model["w_down"][:n_layers]
    out["gain"] = np.concatenate([model["gain"][:n_layers], model["gain"][-1:]])
    return out
