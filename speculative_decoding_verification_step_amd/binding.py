"""ctypes binding of libspecverify.so (include/spec_verify.h).

Argument marshalling only: torch is used for device memory and the current
HIP stream; every step of the verification runs in the library's kernels.
The library must have been built in-tree; nothing falls back to Python or
CPU code when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = 0, -1, -2, -3, -4
SV_F32, SV_BF16 = 0, 1
SV_LAYOUT_ROW_MAJOR, SV_LAYOUT_TILED = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_sz = ctypes.c_size_t


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spec_verify error {code}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("d", _i32), ("ffn", _i32), ("n_layers", _i32), ("vocab", _i32),
                ("wdtype", _i32), ("layout", _i32), ("rms_eps", ctypes.c_float),
                ("w_up", _vp), ("w_down", _vp), ("gain", _vp), ("w_head", _vp)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", _i32), ("total_ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


EXPORTS = {
    "spec_verify_abi_version": (_i32, []),
    "spec_verify_packed_elems": (_sz, [_i32, _i32]),
    "spec_verify_pack_weights": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "sv_model_create": (ctypes.c_int, [ctypes.POINTER(ModelDesc), ctypes.POINTER(_vp)]),
    "sv_model_destroy": (None, [_vp]),
    "spec_verify_forward_workspace_bytes": (_sz, [_vp, _i32]),
    "spec_verify_accept_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "spec_verify_workspace_bytes": (_sz, [_vp, _i32, _i32]),
    "spec_verify_forward": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "spec_verify_accept": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, ctypes.c_float, _u64,
                                          _u32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_accept_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, ctypes.c_float,
                                                  _u64, _u32, _vp, _vp, _vp, _vp, _vp]),
    "spec_verify_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_float, _u64, _u32,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_last_error": (ctypes.c_char_p, []),
    "spec_verify_profile_begin": (ctypes.c_int, [_i32]),
    "spec_verify_profile_pause": (ctypes.c_int, [_i32]),
    "spec_verify_profile_end": (ctypes.c_int, [ctypes.POINTER(KernelTime), _i32,
                                               ctypes.POINTER(_i32)]),
    "spec_verify_choose_k": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp]),
    "spec_verify_attention_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "spec_verify_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _vp]),
    "spec_verify_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                             _i32, _i32, ctypes.c_float, _vp, _vp, _sz, _vp]),
    "spec_verify_kv_commit": (ctypes.c_int, [_vp, _vp, _i32, _vp]),
    "sv_kv_pool_create": (ctypes.c_int, [_i32, ctypes.POINTER(_vp)]),
    "sv_kv_pool_destroy": (None, [_vp]),
    "sv_kv_pool_free_blocks": (_i32, [_vp]),
    "sv_kv_pool_reserve": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32]),
    "sv_kv_pool_trim": (ctypes.c_int, [_vp, _vp, _vp, _i32]),
    "spec_verify_window_k": (_i32, [_vp, _i32, _i32, ctypes.c_float, _i32, _i32]),
    "sv_moe_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(_vp)]),
    "sv_moe_destroy": (None, [_vp]),
    "spec_verify_moe_workspace_bytes": (_sz, [_vp, _i32]),
    "spec_verify_moe_forward": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_embed": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _vp]),
    "spec_verify_sample_workspace_bytes": (_sz, [_i32, _i32]),
    "spec_verify_sample": (ctypes.c_int, [_vp, _i32, _i32, ctypes.c_float, _u64, _u32, _i32, _vp,
                                          _i32, _vp, _sz, _vp]),
    "spec_verify_draft_workspace_bytes": (_sz, [_vp, _i32]),
    "spec_verify_draft": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, ctypes.c_float, _u64, _u32, _vp,
                                         _vp, _vp, _sz, _vp]),
    "spec_verify_cycle_workspace_bytes": (_sz, [_vp, _vp, _i32, _i32]),
    "spec_verify_cycle": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_float, _u64, _u32,
                                         _vp, _vp, _vp, _sz, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first with "
                "`python -m speculative_decoding_verification_step_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != SV_OK:
        raise SpecVerifyError(rc, lib().spec_verify_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A caller-owned workspace buffer (256-byte aligned by torch's allocator)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


def pack(w, stream=None):
    """Tiled copy of bf16 row-major weights: w is [rows, cols] or a stack
    [count, rows, cols]; returns a flat bf16 tensor of
    count * spec_verify_packed_elems(rows, cols) elements."""
    _need(w, "w", torch.bfloat16)
    if w.dim() == 2:
        count, rows, cols = 1, w.shape[0], w.shape[1]
    elif w.dim() == 3:
        count, rows, cols = w.shape
    else:
        raise ValueError("w must be 2-D or 3-D")
    n = int(lib().spec_verify_packed_elems(rows, cols))
    if n == 0:
        raise ValueError(f"cannot pack a [{rows}, {cols}] matrix (cols must be a multiple of 32)")
    out = torch.empty(max(count * n, 1), dtype=torch.bfloat16, device=w.device)
    if count:
        _check(lib().spec_verify_pack_weights(_ptr(w), _ptr(out), rows, cols, count, _stream(stream)))
    return out


class Model:
    """Borrowed view of target weights already resident on the GPU.

    Row-major layout: w_up [L, ffn, d], w_down [L, d, ffn], w_head [V, d]
    (bfloat16 or float32).  Tiled layout (bf16; see ``pack``): pass the packed
    tensors with ``layout="tiled"`` and the shapes in ``dims = (L, d, ffn, V)``.
    gain [L+1, d] float32.  The tensors are kept referenced for the model's
    lifetime.  ``Model.packed(...)`` packs row-major bf16 weights first."""

    def __init__(self, w_up, w_down, gain, w_head, rms_eps: float = 1e-5, layout: str = "row",
                 dims=None):
        dt = w_head.dtype
        if dt not in (torch.bfloat16, torch.float32):
            raise ValueError("weights must be bfloat16 or float32")
        if layout == "row":
            V, d = w_head.shape
            L, ffn = w_up.shape[0], w_up.shape[1]
            _need(w_up, "w_up", dt, (L, ffn, d))
            _need(w_down, "w_down", dt, (L, d, ffn))
            _need(w_head, "w_head", dt, (V, d))
            lay = SV_LAYOUT_ROW_MAJOR
        elif layout == "tiled":
            L, d, ffn, V = dims
            pe = lambda r, c: int(lib().spec_verify_packed_elems(r, c))
            _need(w_up, "w_up", torch.bfloat16)
            _need(w_down, "w_down", torch.bfloat16)
            _need(w_head, "w_head", torch.bfloat16)
            if L and (w_up.numel() < L * pe(ffn, d) or w_down.numel() < L * pe(d, ffn)):
                raise ValueError("packed block weights too small")
            if w_head.numel() < pe(V, d):
                raise ValueError("packed head too small")
            lay = SV_LAYOUT_TILED
        else:
            raise ValueError("layout must be 'row' or 'tiled'")
        _need(gain, "gain", torch.float32, (L + 1, d))
        self._keep = (w_up, w_down, gain, w_head)
        self.d, self.ffn, self.n_layers, self.vocab, self.dtype = d, ffn, L, V, dt
        self.layout = layout
        desc = ModelDesc(d, ffn, L, V, SV_BF16 if dt == torch.bfloat16 else SV_F32, lay, rms_eps,
                         w_up.data_ptr() if L else None, w_down.data_ptr() if L else None,
                         gain.data_ptr(), w_head.data_ptr())
        h = ctypes.c_void_p()
        _check(lib().sv_model_create(ctypes.byref(desc), ctypes.byref(h)))
        self._h = h

    @classmethod
    def packed(cls, w_up, w_down, gain, w_head, rms_eps: float = 1e-5):
        """Pack row-major bf16 weights into the tiled layout and wrap them."""
        L, ffn, d = w_up.shape
        V = w_head.shape[0]
        up, down, hd = pack(w_up), pack(w_down), pack(w_head)
        return cls(up, down, gain, hd, rms_eps, layout="tiled", dims=(L, d, ffn, V))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.sv_model_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def forward_workspace_bytes(self, M: int) -> int:
        return int(lib().spec_verify_forward_workspace_bytes(self._h, M))

    def workspace_bytes(self, B: int, K: int) -> int:
        return int(lib().spec_verify_workspace_bytes(self._h, B, K))

    def forward(self, hidden, logits=None, ws=None, stream=None):
        """Logits [M, V] fp32 of hidden [M, d] fp32."""
        M = hidden.shape[0]
        _need(hidden, "hidden", torch.float32, (M, self.d))
        if logits is None:
            logits = torch.empty((M, self.vocab), dtype=torch.float32, device=hidden.device)
        _need(logits, "logits", torch.float32, (M, self.vocab))
        if ws is None:
            ws = workspace(self.forward_workspace_bytes(M), hidden.device)
        _check(lib().spec_verify_forward(self._h, _ptr(hidden), M, _ptr(logits), _ptr(ws),
                                         ws.numel(), _stream(stream)))
        return logits

    def step(self, hidden, draft_logits, draft_tokens, B: int, K: int, temperature: float,
             seed: int, step: int, logits=None, out_tokens=None, accept_len=None,
             p_at=None, q_at=None, ws=None, stream=None):
        """The whole verification step; returns (logits, out_tokens, accept_len)."""
        M = B * (K + 1)
        dev = hidden.device
        _need(hidden, "hidden", torch.float32, (M, self.d))
        if draft_logits is not None:
            _need(draft_logits, "draft_logits", torch.float32, (B, K, self.vocab))
        if draft_tokens is not None:
            _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
        if logits is None:
            logits = torch.empty((M, self.vocab), dtype=torch.float32, device=dev)
        if out_tokens is None:
            out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        if accept_len is None:
            accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
        _need(logits, "logits", torch.float32, (M, self.vocab))
        _need(out_tokens, "out_tokens", torch.int32, (B, K + 1))
        _need(accept_len, "accept_len", torch.int32, (B,))
        for t, n in ((p_at, "p_at"), (q_at, "q_at")):
            if t is not None:
                _need(t, n, torch.float32, (B, K))
        if ws is None:
            ws = workspace(self.workspace_bytes(B, K), dev)
        _check(lib().spec_verify_step(self._h, _ptr(hidden), _ptr(draft_logits), _ptr(draft_tokens),
                                      B, K, float(temperature), int(seed), int(step), _ptr(logits),
                                      _ptr(out_tokens), _ptr(accept_len), _ptr(p_at), _ptr(q_at),
                                      _ptr(ws), ws.numel(), _stream(stream)))
        return logits, out_tokens, accept_len


    def draft_workspace_bytes(self, B: int) -> int:
        return int(lib().spec_verify_draft_workspace_bytes(self._h, B))

    def draft(self, table, cur, K: int, temperature: float, seed: int, step: int,
              draft_tokens=None, draft_logits=None, ws=None, stream=None):
        """The draft loop with this model as the drafter (include/spec_verify_cycle.h):
        table [V, d] fp32 embedding rows, cur [B] int32 current tokens.
        Returns (draft_tokens [B, K] int32, draft_logits [B, K, V] fp32)."""
        B = cur.shape[0]
        dev = cur.device
        _need(table, "table", torch.float32, (self.vocab, self.d))
        _need(cur, "cur", torch.int32, (B,))
        if draft_tokens is None:
            draft_tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
        if draft_logits is None:
            draft_logits = torch.empty((B, K, self.vocab), dtype=torch.float32, device=dev)
        _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
        _need(draft_logits, "draft_logits", torch.float32, (B, K, self.vocab))
        if ws is None:
            ws = workspace(self.draft_workspace_bytes(B), dev)
        _check(lib().spec_verify_draft(self._h, _ptr(table), _ptr(cur), B, K, float(temperature),
                                       int(seed), int(step), _ptr(draft_tokens), _ptr(draft_logits),
                                       _ptr(ws), ws.numel(), _stream(stream)))
        return draft_tokens, draft_logits


def embed(table, tokens, hidden=None, stream=None):
    """hidden [n, d] fp32 = table[tokens] (zero rows for tokens outside [0, V))."""
    V, d = table.shape
    n = tokens.shape[0]
    _need(table, "table", torch.float32, (V, d))
    _need(tokens, "tokens", torch.int32, (n,))
    if hidden is None:
        hidden = torch.empty((n, d), dtype=torch.float32, device=table.device)
    _need(hidden, "hidden", torch.float32, (n, d))
    _check(lib().spec_verify_embed(_ptr(table), V, d, _ptr(tokens), n, _ptr(hidden), _stream(stream)))
    return hidden


def sample_workspace_bytes(B: int, V: int) -> int:
    return int(lib().spec_verify_sample_workspace_bytes(B, V))


def sample(logits, temperature: float, seed: int, step: int, slot: int, tokens=None,
           out_stride: int = 1, ws=None, stream=None):
    """One token per row of logits [B, V]: tokens[b * out_stride] drawn from
    softmax(logits[b] / T) with Philox counter (b, slot, 2, step)."""
    B, V = logits.shape
    _need(logits, "logits", torch.float32, (B, V))
    if tokens is None:
        tokens = torch.empty((B * out_stride,), dtype=torch.int32, device=logits.device)
    _need(tokens, "tokens", torch.int32)
    if tokens.numel() < (B - 1) * out_stride + 1:
        raise ValueError("tokens too small for B and out_stride")
    if ws is None:
        ws = workspace(sample_workspace_bytes(B, V), logits.device)
    _check(lib().spec_verify_sample(_ptr(logits), B, V, float(temperature), int(seed), int(step),
                                    int(slot), _ptr(tokens), int(out_stride), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return tokens


def cycle_workspace_bytes(target, drafter, B: int, K: int) -> int:
    return int(lib().spec_verify_cycle_workspace_bytes(target.handle,
                                                       drafter.handle if drafter else None, B, K))


def cycle(target, drafter, table, cur, K: int, temperature: float, seed: int, step: int,
          out_tokens=None, accept_len=None, ws=None, stream=None):
    """One speculative cycle (include/spec_verify_cycle.h): draft K tokens,
    verify the K + 1 positions, move cur [B] int32 (in place) to the last
    token emitted.  K = 0 is one step of plain decoding (drafter may be None).
    Returns (out_tokens [B, K+1], accept_len [B])."""
    B = cur.shape[0]
    dev = cur.device
    _need(table, "table", torch.float32, (target.vocab, target.d))
    _need(cur, "cur", torch.int32, (B,))
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, (B, K + 1))
    _need(accept_len, "accept_len", torch.int32, (B,))
    if ws is None:
        ws = workspace(cycle_workspace_bytes(target, drafter, B, K), dev)
    _check(lib().spec_verify_cycle(target.handle, drafter.handle if drafter else None, _ptr(table),
                                   _ptr(cur), B, K, float(temperature), int(seed), int(step),
                                   _ptr(out_tokens), _ptr(accept_len), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return out_tokens, accept_len


def accept_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(lib().spec_verify_accept_workspace_bytes(B, K, V))


def accept(target_logits, draft_logits, draft_tokens, temperature: float, seed: int, step: int,
           out_tokens=None, accept_len=None, p_at=None, q_at=None, ws=None, stream=None):
    """Rejection sampling alone: target_logits [B, K+1, V], draft_logits
    [B, K, V] (or None at T = 0 / K = 0), draft_tokens [B, K] int32.
    Returns (out_tokens [B, K+1], accept_len [B])."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, K1, V))
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, (B, K, V))
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(accept_workspace_bytes(B, K, V), dev)
    _check(lib().spec_verify_accept(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
                                    B, K, V, float(temperature), int(seed), int(step),
                                    _ptr(out_tokens), _ptr(accept_len), _ptr(p_at), _ptr(q_at),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    return out_tokens, accept_len


def accept_noalloc(target_logits, draft_logits, draft_tokens, temperature: float, seed: int,
                   step: int, out_tokens, accept_len, p_at=None, q_at=None, stream=None):
    """``accept`` through the entry point that allocates nothing (its scratch is
    the library's static per-device array): the outputs must be passed in."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits", torch.float32, (B, K1, V))
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, (B, K, V))
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _need(out_tokens, "out_tokens", torch.int32, (B, K1))
    _need(accept_len, "accept_len", torch.int32, (B,))
    _check(lib().spec_verify_accept_noalloc(_ptr(target_logits), _ptr(draft_logits),
                                            _ptr(draft_tokens), B, K, V, float(temperature),
                                            int(seed), int(step), _ptr(out_tokens),
                                            _ptr(accept_len), _ptr(p_at), _ptr(q_at),
                                            _stream(stream)))
    return out_tokens, accept_len


def profile_begin(max_launches: int = 65536):
    _check(lib().spec_verify_profile_begin(max_launches))


def profile_pause(paused: bool):
    _check(lib().spec_verify_profile_pause(1 if paused else 0))


def profile_end(cap: int = 64):
    """Stop per-launch timing; returns {name: (launches, total_ms, bytes, flops)}."""
    arr = (KernelTime * cap)()
    n = _i32(0)
    _check(lib().spec_verify_profile_end(arr, cap, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms, arr[i].bytes, arr[i].flops)
            for i in range(min(n.value, cap))}


def choose_k(m_rows, t_verif, al, batch, t_draft=None):
    """Goodput-optimal draft length per batch size (host arrays; see
    include/spec_verify_kselect.h).  Returns (k [n_b] int32, goodput [n_b])."""
    m = np.ascontiguousarray(m_rows, dtype=np.int32)
    t = np.ascontiguousarray(t_verif, dtype=np.float64)
    a = np.ascontiguousarray(al, dtype=np.float64)
    b = np.ascontiguousarray(batch, dtype=np.int32)
    d = None if t_draft is None else np.ascontiguousarray(t_draft, dtype=np.float64)
    if d is not None and d.shape != (len(b), len(a)):
        raise ValueError(f"t_draft must be [{len(b)}, {len(a)}], got {d.shape}")
    if len(t) != len(m):
        raise ValueError("m_rows and t_verif differ in length")
    k = np.empty(len(b), np.int32)
    g = np.empty(len(b), np.float64)
    _check(lib().spec_verify_choose_k(m.ctypes.data, t.ctypes.data, len(m), a.ctypes.data, len(a),
                                      b.ctypes.data, len(b),
                                      None if d is None else d.ctypes.data,
                                      k.ctypes.data, g.ctypes.data))
    return k, g


def window_k(accept_len, window: int = 10, threshold: float = 1.5, k_high: int = 5,
             k_low: int = 2) -> int:
    """Speculation window from recent acceptance lengths (host array)."""
    a = np.ascontiguousarray(accept_len, dtype=np.int32)
    r = int(lib().spec_verify_window_k(a.ctypes.data if len(a) else None, len(a), window,
                                       float(threshold), k_high, k_low))
    if r < 0:
        _check(r)
    return r


# ---- paged attention of the verified positions (include/spec_verify_attn.h) ----
KV_BLOCK = 32


def _bf16(t, name, shape):
    _need(t, name, torch.bfloat16, shape)


def attention_workspace_bytes(B: int, T: int, Hq: int, Hkv: int, head_dim: int,
                              max_blocks: int) -> int:
    return int(lib().spec_verify_attention_workspace_bytes(B, T, Hq, Hkv, head_dim, max_blocks))


def kv_append(k_new, v_new, k_cache, v_cache, block_table, ctx_len, stream=None):
    """Write k_new / v_new [B, T, Hkv, Dh] (bf16) at positions ctx_len[b] + t."""
    B, T, Hkv, Dh = k_new.shape
    nb = k_cache.shape[0]
    mb = block_table.shape[1]
    _bf16(k_new, "k_new", (B, T, Hkv, Dh))
    _bf16(v_new, "v_new", (B, T, Hkv, Dh))
    _bf16(k_cache, "k_cache", (nb, Hkv, KV_BLOCK, Dh))
    _bf16(v_cache, "v_cache", (nb, Hkv, Dh, KV_BLOCK))
    _need(block_table, "block_table", torch.int32, (B, mb))
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    _check(lib().spec_verify_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_table), _ptr(ctx_len), B, T, Hkv, Dh, mb, nb,
                                       _stream(stream)))


def attention(q, k_cache, v_cache, block_table, ctx_len, scale: float, out=None, ws=None,
              stream=None):
    """Causal attention of q [B, T, Hq, Dh] (bf16) over the paged cache;
    returns out [B, T, Hq, Dh] fp32."""
    B, T, Hq, Dh = q.shape
    nb, Hkv = k_cache.shape[:2]
    mb = block_table.shape[1]
    _bf16(q, "q", (B, T, Hq, Dh))
    _bf16(k_cache, "k_cache", (nb, Hkv, KV_BLOCK, Dh))
    _bf16(v_cache, "v_cache", (nb, Hkv, Dh, KV_BLOCK))
    _need(block_table, "block_table", torch.int32, (B, mb))
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, T, Hq, Dh), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, T, Hq, Dh))
    if ws is None:
        n = attention_workspace_bytes(B, T, Hq, Hkv, Dh, mb)
        ws = workspace(n, q.device) if n else None
    _check(lib().spec_verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(ctx_len), B, T, Hq, Hkv, Dh, mb, nb, float(scale),
                                       _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream)))
    return out


def kv_commit(ctx_len, accept_len, stream=None):
    """ctx_len[b] += accept_len[b] (AL >= 1) on the device."""
    B = ctx_len.shape[0]
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    _need(accept_len, "accept_len", torch.int32, (B,))
    _check(lib().spec_verify_kv_commit(_ptr(ctx_len), _ptr(accept_len), B, _stream(stream)))


class KVPool:
    """Host free list of physical KV blocks (sv_kv_pool)."""

    def __init__(self, num_blocks: int):
        h = _vp()
        _check(lib().sv_kv_pool_create(num_blocks, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.sv_kv_pool_destroy(self._h)
            self._h = None

    @property
    def free_blocks(self) -> int:
        return int(lib().sv_kv_pool_free_blocks(self._h))

    def reserve(self, row: np.ndarray, n_blocks: int, tokens: int) -> int:
        """Grow a host int32 table row (n_blocks in use) to cover `tokens`."""
        assert row.dtype == np.int32 and row.flags.c_contiguous
        n = _i32(n_blocks)
        _check(lib().sv_kv_pool_reserve(self._h, row.ctypes.data, ctypes.byref(n), len(row), tokens))
        return n.value

    def trim(self, row: np.ndarray, n_blocks: int, tokens: int) -> int:
        """Return the row's blocks past `tokens` positions; the new count."""
        assert row.dtype == np.int32 and row.flags.c_contiguous
        n = _i32(n_blocks)
        _check(lib().sv_kv_pool_trim(self._h, row.ctypes.data, ctypes.byref(n), tokens))
        return n.value


# ---- mixture-of-experts target (include/spec_verify_moe.h) --------------------
class MoEDesc(ctypes.Structure):
    _fields_ = [("d", _i32), ("ffn", _i32), ("n_experts", _i32), ("top_k", _i32),
                ("n_layers", _i32), ("vocab", _i32), ("rms_eps", ctypes.c_float),
                ("w_router", _vp), ("w_up", _vp), ("w_down", _vp), ("gain", _vp), ("w_head", _vp)]


class MoEModel:
    """Borrowed view of packed MoE weights on the GPU (bf16, tiled).  Use
    ``MoEModel.packed`` to pack row-major weights: w_router [L, E, d],
    w_up [L, E, ffn, d], w_down [L, E, d, ffn], w_head [V, d], gain [L+1, d]."""

    def __init__(self, w_router, w_up, w_down, gain, w_head, dims, top_k: int,
                 rms_eps: float = 1e-5):
        L, E, d, ffn, V = dims
        _need(gain, "gain", torch.float32, (L + 1, d))
        for t, name in ((w_router, "w_router"), (w_up, "w_up"), (w_down, "w_down"), (w_head, "w_head")):
            _need(t, name, torch.bfloat16)
        self._keep = (w_router, w_up, w_down, gain, w_head)
        self.n_layers, self.n_experts, self.d, self.ffn, self.vocab = L, E, d, ffn, V
        self.top_k = top_k
        desc = MoEDesc(d, ffn, E, top_k, L, V, rms_eps, _ptr(w_router), _ptr(w_up), _ptr(w_down),
                       _ptr(gain), _ptr(w_head))
        h = _vp()
        _check(lib().sv_moe_create(ctypes.addressof(desc), ctypes.byref(h)))
        self._h = h

    @classmethod
    def packed(cls, w_router, w_up, w_down, gain, w_head, top_k: int, rms_eps: float = 1e-5):
        L, E, d = w_router.shape
        ffn = w_up.shape[2]
        V = w_head.shape[0]
        return cls(pack(w_router), pack(w_up.reshape(L * E, ffn, d)), pack(w_down.reshape(L * E, d, ffn)),
                   gain, pack(w_head), (L, E, d, ffn, V), top_k, rms_eps)

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.sv_moe_destroy(self._h)
            self._h = None

    def workspace_bytes(self, M: int) -> int:
        return int(lib().spec_verify_moe_workspace_bytes(self._h, M))

    def forward(self, hidden, logits=None, active=None, ws=None, stream=None):
        """Logits [M, V] fp32; ``active`` (int32 [n_layers] on the GPU) gets the
        distinct experts each block used."""
        M = hidden.shape[0]
        _need(hidden, "hidden", torch.float32, (M, self.d))
        if logits is None:
            logits = torch.empty((M, self.vocab), dtype=torch.float32, device=hidden.device)
        _need(logits, "logits", torch.float32, (M, self.vocab))
        if active is not None:
            _need(active, "active", torch.int32, (self.n_layers,))
        if ws is None:
            ws = workspace(self.workspace_bytes(M), hidden.device)
        _check(lib().spec_verify_moe_forward(self._h, _ptr(hidden), M, _ptr(logits), _ptr(active),
                                             _ptr(ws), ws.numel(), _stream(stream)))
        return logits
