"""Thin Python binding over libec.so (include/ec.h), same names as the C ABI.

PyTorch is used only for device memory and streams: every computation of the
denoising step runs in the library's HIP kernels. Tensors are passed as raw
device pointers; shapes and dtypes are checked here before the call, and the
library checks them again.
"""
from __future__ import annotations

import ctypes as C
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import check, load

_DT = {torch.float32: _lib.EC_F32, torch.bfloat16: _lib.EC_BF16}
_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------- kernels
def ec_entropy_max(logits: torch.Tensor, sel: Optional[torch.Tensor] = None, stream=None,
                   workspace: Optional[torch.Tensor] = None, out=None):
    """Per-row softmax entropy (nats), argmax, max-probability and E = max entropy over sel.

    logits: [rows, V] (row stride may exceed V), float32 or bfloat16, on the GPU.
    Returns (entropy f32[rows], argmax i32[rows], maxprob f32[rows], emax f32[1]); ``out``
    may pass those four tensors in to be filled instead of allocated.
    """
    lib = load()
    _need_cuda(logits, sel)
    if logits.dim() != 2 or (logits.shape[0] > 0 and logits.stride(1) != 1):
        raise ValueError("logits must be 2-D with unit column stride")
    rows, V = logits.shape
    dev = logits.device
    if out is not None:
        H, a, c, e = out
        if (H.numel() < rows or a.numel() < rows or c.numel() < rows or e.numel() < 1
                or (H.dtype, a.dtype, c.dtype, e.dtype) != (torch.float32, torch.int32, torch.float32, torch.float32)):
            raise ValueError("out: need float32[rows], int32[rows], float32[rows], float32[1]")
    else:
        H = torch.empty(rows, dtype=torch.float32, device=dev)
        a = torch.empty(rows, dtype=torch.int32, device=dev)
        c = torch.empty(rows, dtype=torch.float32, device=dev)
        e = torch.empty(1, dtype=torch.float32, device=dev)
    if sel is not None:
        sel = sel.to(torch.int32).contiguous()
    ws_bytes = lib.ec_entropy_max_workspace_size(rows, V)
    ws = workspace if workspace is not None else _workspace(ws_bytes, dev)
    stride = logits.stride(0) if rows > 0 else V
    check(lib.ec_entropy_max(_ptr(logits), _dtype(logits), rows, V, stride, _ptr(sel),
                             0 if sel is None else sel.numel(), _ptr(H), _ptr(a), _ptr(c), _ptr(e),
                             _ptr(ws), ws.numel(), _stream(stream)), "ec_entropy_max")
    return H, a, c, e


def ec_entropy_max_noalloc(logits: torch.Tensor, sel: Optional[torch.Tensor] = None, stream=None, out=None):
    """ec_entropy_max without a workspace (the library's own device scratch array): for
    callers that cannot allocate. Same arguments and results as ec_entropy_max; ``out``
    (four tensors as there) avoids allocating the outputs too."""
    lib = load()
    _need_cuda(logits, sel)
    if logits.dim() != 2 or (logits.shape[0] > 0 and logits.stride(1) != 1):
        raise ValueError("logits must be 2-D with unit column stride")
    rows, V = logits.shape
    dev = logits.device
    if out is not None:
        H, a, c, e = out
        if (H.numel() < rows or a.numel() < rows or c.numel() < rows or e.numel() < 1
                or (H.dtype, a.dtype, c.dtype, e.dtype) != (torch.float32, torch.int32, torch.float32, torch.float32)):
            raise ValueError("out: need float32[rows], int32[rows], float32[rows], float32[1]")
    else:
        H = torch.empty(rows, dtype=torch.float32, device=dev)
        a = torch.empty(rows, dtype=torch.int32, device=dev)
        c = torch.empty(rows, dtype=torch.float32, device=dev)
        e = torch.empty(1, dtype=torch.float32, device=dev)
    if sel is not None and sel.dtype != torch.int32:
        raise ValueError("sel must be int32 (no conversion is made here)")
    stride = logits.stride(0) if rows > 0 else V
    check(lib.ec_entropy_max_noalloc(_ptr(logits), _dtype(logits), rows, V, stride, _ptr(sel),
                                     0 if sel is None else sel.numel(), _ptr(H), _ptr(a), _ptr(c), _ptr(e),
                                     _stream(stream)), "ec_entropy_max_noalloc")
    return H, a, c, e


def ec_cache_scatter(k_cache: torch.Tensor, v_cache: torch.Tensor, k_rows: torch.Tensor,
                     v_rows: torch.Tensor, idx: torch.Tensor, stream=None) -> None:
    """k_cache[idx[i]] = k_rows[i]; v_cache[idx[i]] = v_rows[i] (in place)."""
    lib = load()
    _need_cuda(k_cache, v_cache, k_rows, v_rows, idx)
    for t in (k_cache, v_cache, k_rows, v_rows):
        if not t.is_contiguous() or t.dim() != 2:
            raise ValueError("cache and rows must be contiguous 2-D tensors")
    if k_cache.shape != v_cache.shape or k_rows.shape != v_rows.shape or k_rows.shape[1] != k_cache.shape[1]:
        raise ValueError("shape mismatch")
    if len({k_cache.dtype, v_cache.dtype, k_rows.dtype, v_rows.dtype}) != 1:
        raise ValueError("dtype mismatch")
    idx = idx.to(torch.int32).contiguous()
    if idx.numel() != k_rows.shape[0]:
        raise ValueError("idx length must equal the number of rows")
    check(lib.ec_cache_scatter(_ptr(k_cache), _ptr(v_cache), k_cache.shape[0], k_cache.shape[1],
                               _dtype(k_cache), _ptr(k_rows), _ptr(v_rows), _ptr(idx), idx.numel(),
                               _stream(stream)), "ec_cache_scatter")


def ec_partial_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, n_heads: int,
                    head_dim: int, scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """Bidirectional attention of q [r, H*D] over all rows of k/v_cache [L, H*D]."""
    lib = load()
    _need_cuda(q, k_cache, v_cache)
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous() or t.dim() != 2 or t.shape[1] != n_heads * head_dim:
            raise ValueError("q and caches must be contiguous [rows, n_heads*head_dim]")
    r, L = q.shape[0], k_cache.shape[0]
    if v_cache.shape[0] != L:
        raise ValueError("k/v cache length mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = torch.empty_like(q)
    ws = _workspace(lib.ec_partial_attn_workspace_size(r, L, n_heads, head_dim), q.device)
    check(lib.ec_partial_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), r, L, n_heads, head_dim,
                              float(scale), _dtype(q), _ptr(out), _ptr(ws), ws.numel(),
                              _stream(stream)), "ec_partial_attn")
    return out


def ec_partial_attn_plan(r: int, seq_len: int, n_heads: int, head_dim: int = 128) -> Tuple[int, int]:
    """(queries per workgroup, key splits) that the bf16 ec_partial_attn launches for
    these sizes (host only)."""
    lib = load()
    qt, sp = C.c_int32(0), C.c_int32(0)
    check(lib.ec_partial_attn_plan(r, seq_len, n_heads, head_dim, C.byref(qt), C.byref(sp)),
          "ec_partial_attn_plan")
    return qt.value, sp.value


def ec_rope_table(max_pos: int, head_dim: int, base: float = 10000.0, device="cuda", stream=None):
    lib = load()
    c = torch.empty(max_pos, head_dim // 2, dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    check(lib.ec_rope_table(_ptr(c), _ptr(s), max_pos, head_dim, float(base), _stream(stream)),
          "ec_rope_table")
    return c, s


# ---------------------------------------------------------------------- model / cache
def _to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def pack_weights(shape, wqkv: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, stream=None):
    """ec_pack_weights: plain [3d, d] and [F, d] x2 device matrices -> packed
    (wqkv [3d, d], gate/up [2F, d]) for the MFMA kernels."""
    lib = load()
    d, F = shape.d_model, shape.ffn_dim
    for t, rows in ((wqkv, 3 * d), (w_gate, F), (w_up, F)):
        assert t.is_contiguous() and tuple(t.shape) == (rows, d), "pack_weights: bad matrix shape"
    qp = torch.empty_like(wqkv)
    gu = torch.empty(2 * F, d, dtype=w_gate.dtype, device=w_gate.device)
    dt = _lib.EC_BF16 if wqkv.dtype == torch.bfloat16 else _lib.EC_F32
    check(lib.ec_pack_weights(dt, d, shape.head_dim, F, _ptr(wqkv), _ptr(w_gate), _ptr(w_up),
                              _ptr(qp), _ptr(gu), _stream(stream)), "ec_pack_weights")
    return qp, gu


class DeviceModel:
    """Weights on the GPU plus the ec_model_desc that points at them."""

    def __init__(self, shape, embed, layers: List[dict], final_norm, lm_head, rope_max_pos: int,
                 device="cuda"):
        lib = load()
        self.shape = shape
        self.device = torch.device(device)
        self.embed, self.layers, self.final_norm, self.lm_head = embed, layers, final_norm, lm_head
        self.rope_cos, self.rope_sin = ec_rope_table(rope_max_pos, shape.head_dim, shape.rope_base,
                                                     self.device)
        n = len(layers)
        if shape.dtype == "bf16":
            # the MFMA kernels read the packed layout; repack each layer on the device
            # in place of the plain matrices (ec_pack_weights)
            for lw in layers:
                lw["wqkv"], lw["w_gate"] = pack_weights(shape, lw["wqkv"], lw["w_gate"], lw["w_up"])
                lw["w_up"] = None
        self._lw = (_lib.ec_layer_weights * n)()
        for i, lw in enumerate(layers):
            for name in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
                setattr(self._lw[i], name, lw[name].data_ptr() if lw[name] is not None else None)
        d = _lib.ec_model_desc()
        d.struct_size = C.sizeof(_lib.ec_model_desc)
        d.dtype = _lib.EC_BF16 if shape.dtype == "bf16" else _lib.EC_F32
        d.n_layers, d.d_model, d.n_heads = n, shape.d_model, shape.n_heads
        d.head_dim, d.ffn_dim, d.vocab = shape.head_dim, shape.ffn_dim, shape.vocab
        d.rms_eps = shape.rms_eps
        d.embed, d.final_norm, d.lm_head = embed.data_ptr(), final_norm.data_ptr(), lm_head.data_ptr()
        d.layers = C.cast(self._lw, C.POINTER(_lib.ec_layer_weights))
        d.rope_cos, d.rope_sin, d.rope_max_pos = self.rope_cos.data_ptr(), self.rope_sin.data_ptr(), rope_max_pos
        d.weight_layout = _lib.EC_LAYOUT_PACKED if shape.dtype == "bf16" else _lib.EC_LAYOUT_PLAIN
        self.desc = d
        _ = lib

    @property
    def torch_dtype(self):
        return _TORCH_DT[self.shape.dtype]

    @classmethod
    def from_host(cls, weights, rope_max_pos: int, device="cuda") -> "DeviceModel":
        """Upload seeded host weights (``synth.ModelWeights``)."""
        dt = weights.shape.dtype
        up = lambda a: _to_device(a, dt, device)
        layers = [{k: up(v) for k, v in lw.items()} for lw in weights.layers]
        return cls(weights.shape, up(weights.embed), layers, up(weights.final_norm),
                   up(weights.lm_head), rope_max_pos, device)


class KVCache:
    """Per-layer K and V [L, d] buffers plus the ec_cache_desc."""

    def __init__(self, model: DeviceModel, seq_len: int):
        n, d = len(model.layers), model.shape.d_model
        self.k = [torch.zeros(seq_len, d, dtype=model.torch_dtype, device=model.device) for _ in range(n)]
        self.v = [torch.zeros(seq_len, d, dtype=model.torch_dtype, device=model.device) for _ in range(n)]
        self._kp = (C.c_void_p * n)(*[t.data_ptr() for t in self.k])
        self._vp = (C.c_void_p * n)(*[t.data_ptr() for t in self.v])
        c = _lib.ec_cache_desc()
        c.struct_size = C.sizeof(_lib.ec_cache_desc)
        c.seq_len = seq_len
        c.k = C.cast(self._kp, C.POINTER(C.c_void_p))
        c.v = C.cast(self._vp, C.POINTER(C.c_void_p))
        self.desc = c
        self.seq_len = seq_len


def ec_forward(model: DeviceModel, cache: KVCache, tokens: torch.Tensor, rows: torch.Tensor,
               out_idx: torch.Tensor, want_hidden: bool = False, stream=None,
               workspace: Optional[torch.Tensor] = None):
    """Forward over positions ``rows`` against ``cache``; logits for rows[out_idx].

    Returns (logits [n_out, V], hidden [n_rows, d] fp32 or None).
    """
    lib = load()
    dev = model.device
    tokens = tokens.to(torch.int32).contiguous()
    rows = rows.to(torch.int32).contiguous()
    out_idx = out_idx.to(torch.int32).contiguous()
    n_rows, n_out = rows.numel(), out_idx.numel()
    logits = torch.empty(n_out, model.shape.vocab, dtype=model.torch_dtype, device=dev)
    hidden = torch.empty(n_rows, model.shape.d_model, dtype=torch.float32, device=dev) if want_hidden else None
    need = lib.ec_forward_workspace_size(C.byref(model.desc), max(n_rows, 1), n_out, cache.seq_len)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, dev)
    check(lib.ec_forward(C.byref(model.desc), C.byref(cache.desc), _ptr(tokens), _ptr(rows), n_rows,
                         _ptr(out_idx), n_out, _ptr(logits), _ptr(hidden), _ptr(ws), ws.numel(),
                         _stream(stream)), "ec_forward")
    return logits, hidden


# ---------------------------------------------------------------------- decoding
@dataclass
class StepOut:
    status: int
    refreshed: bool
    rows: int
    n_cand: int
    refresh_next: bool
    emax: float
    positions: List[int]
    ids: List[int]
    entropy: List[float]
    maxprob: List[float]


class Decoder:
    """One sequence's EntropyCache decoding state, driven by ec_step."""

    def __init__(self, model: DeviceModel, seq_len: int, prompt_len: int, tokens_per_step: int,
                 block_len: int, k_recent: int, tau: float, cache: Optional[KVCache] = None,
                 window: bool = False):
        lib = load()
        self.model = model
        dev = model.device
        p = _lib.ec_params()
        p.struct_size = C.sizeof(_lib.ec_params)
        p.tau = float(tau)
        p.k_recent, p.tokens_per_step, p.block_len = k_recent, tokens_per_step, block_len
        p.prompt_len, p.seq_len, p.mask_id = prompt_len, seq_len, model.shape.mask_id
        p.candidates = _lib.EC_CAND_WINDOW if window else _lib.EC_CAND_BLOCKS
        self.params = p
        self.cache = cache if cache is not None else KVCache(model, seq_len)
        self.tokens = torch.zeros(seq_len, dtype=torch.int32, device=dev)
        self.masked = torch.zeros(seq_len, dtype=torch.uint8, device=dev)
        self.plan = torch.zeros(lib.ec_state_plan_words(seq_len, k_recent), dtype=torch.int32, device=dev)
        need = lib.ec_step_workspace_size(C.byref(model.desc), C.byref(p))
        if need == 0:
            check(_lib.EC_ERR_ARG, "ec_step_workspace_size")
        self.workspace = _workspace(need, dev)
        st = _lib.ec_state()
        st.struct_size = C.sizeof(_lib.ec_state)
        st.tokens, st.masked, st.plan = self.tokens.data_ptr(), self.masked.data_ptr(), self.plan.data_ptr()
        self.state = st
        self._out = _lib.ec_step_out()
        self._out.struct_size = C.sizeof(_lib.ec_step_out)

    def set_tau(self, tau: float) -> None:
        self.params.tau = float(tau)

    def reset(self, prompt: torch.Tensor, stream=None) -> None:
        """Load prompt ids (the first prompt_len entries of ``prompt`` are used)."""
        P = self.params.prompt_len
        self.tokens[:P].copy_(prompt[:P].to(device=self.tokens.device, dtype=torch.int32))
        check(load().ec_state_reset(C.byref(self.state), C.byref(self.params), _stream(stream)),
              "ec_state_reset")

    @property
    def done(self) -> bool:
        return self.state.n_masked <= 0

    def next_rows(self):
        """Positions the next step recomputes if it is a skip step (R in the plan buffer:
        int32 words from 8 + max(k, 1), state.next_rows of them, ascending)."""
        r0 = 8 + max(self.params.k_recent, 1)
        return self.plan[r0: r0 + self.state.next_rows].cpu().numpy()

    def step(self, stream=None, drift: Optional[torch.Tensor] = None) -> StepOut:
        """One ec_step; with ``drift`` (float32[4 * n_layers] on the GPU) ec_step_probe,
        which also fills per layer the mean / max cosine distance of the recomputed K and V
        rows from their cached values."""
        lib = load()
        if drift is not None:
            if drift.dtype != torch.float32 or drift.numel() < 4 * len(self.model.layers) or not drift.is_cuda:
                raise ValueError("drift: need float32[4 * n_layers] on the GPU")
            rc = lib.ec_step_probe(C.byref(self.model.desc), C.byref(self.cache.desc), C.byref(self.state),
                                   C.byref(self.params), _ptr(self.workspace), self.workspace.numel(),
                                   _stream(stream), C.byref(self._out), _ptr(drift))
        else:
            rc = lib.ec_step(C.byref(self.model.desc), C.byref(self.cache.desc), C.byref(self.state),
                             C.byref(self.params), _ptr(self.workspace), self.workspace.numel(),
                             _stream(stream), C.byref(self._out))
        if rc not in (_lib.EC_OK, _lib.EC_ERR_NAN):
            check(rc, "ec_step_probe" if drift is not None else "ec_step")
        o = self._out
        n = o.n_decoded
        return StepOut(o.status, bool(o.refreshed), o.rows, o.n_cand, bool(o.refresh_next), o.emax,
                       list(o.positions[:n]), list(o.ids[:n]), list(o.entropy[:n]), list(o.maxprob[:n]))

    def run(self, max_steps: Optional[int] = None, stream=None) -> List[StepOut]:
        outs = []
        while not self.done and (max_steps is None or len(outs) < max_steps):
            outs.append(self.step(stream))
        return outs


class BatchDecoder:
    """Several independent sequences of one model stepped together by ec_step_batch:
    one forward over all their rows per step, each sequence deciding refresh or skip
    from its own E."""

    def __init__(self, model: DeviceModel, n_seq: int, seq_len: int, prompt_len: int,
                 tokens_per_step: int, block_len: int, k_recent: int, tau: float, window: bool = False):
        lib = load()
        if not 1 <= n_seq <= _lib.EC_MAX_SEQ:
            raise ValueError(f"n_seq must be in [1, {_lib.EC_MAX_SEQ}]")
        self.model, self.n_seq = model, n_seq
        dev = model.device
        p = _lib.ec_params()
        p.struct_size = C.sizeof(_lib.ec_params)
        p.tau = float(tau)
        p.k_recent, p.tokens_per_step, p.block_len = k_recent, tokens_per_step, block_len
        p.prompt_len, p.seq_len, p.mask_id = prompt_len, seq_len, model.shape.mask_id
        p.candidates = _lib.EC_CAND_WINDOW if window else _lib.EC_CAND_BLOCKS
        self.params = p
        self.caches = [KVCache(model, seq_len) for _ in range(n_seq)]
        words = lib.ec_state_plan_words(seq_len, k_recent)
        self.tokens = [torch.zeros(seq_len, dtype=torch.int32, device=dev) for _ in range(n_seq)]
        self.masked = [torch.zeros(seq_len, dtype=torch.uint8, device=dev) for _ in range(n_seq)]
        self.plans = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(n_seq)]
        self._cd = (_lib.ec_cache_desc * n_seq)(*[c.desc for c in self.caches])
        self.states = (_lib.ec_state * n_seq)()
        self._outs = (_lib.ec_step_out * n_seq)()
        for i in range(n_seq):
            st = self.states[i]
            st.struct_size = C.sizeof(_lib.ec_state)
            st.tokens, st.masked, st.plan = (self.tokens[i].data_ptr(), self.masked[i].data_ptr(),
                                             self.plans[i].data_ptr())
            self._outs[i].struct_size = C.sizeof(_lib.ec_step_out)
        need = lib.ec_step_batch_workspace_size(C.byref(model.desc), n_seq, C.byref(p))
        if need == 0:
            check(_lib.EC_ERR_ARG, "ec_step_batch_workspace_size")
        self.workspace = _workspace(need, dev)

    def set_tau(self, tau: float) -> None:
        self.params.tau = float(tau)

    def reset(self, prompts: Sequence[torch.Tensor], stream=None) -> None:
        """Load each sequence's prompt (the first prompt_len ids of prompts[i])."""
        P = self.params.prompt_len
        for i in range(self.n_seq):
            self.tokens[i][:P].copy_(prompts[i][:P].to(device=self.tokens[i].device, dtype=torch.int32))
            check(load().ec_state_reset(C.byref(self.states[i]), C.byref(self.params), _stream(stream)),
                  "ec_state_reset")

    @property
    def done(self) -> bool:
        return all(self.states[i].n_masked <= 0 for i in range(self.n_seq))

    def step(self, stream=None) -> List[Optional[StepOut]]:
        """One batched step; None for sequences that had nothing left to decode."""
        lib = load()
        active = [self.states[i].n_masked > 0 for i in range(self.n_seq)]
        rc = lib.ec_step_batch(C.byref(self.model.desc), self.n_seq, self._cd, self.states,
                               C.byref(self.params), _ptr(self.workspace), self.workspace.numel(),
                               _stream(stream), self._outs)
        if rc not in (_lib.EC_OK, _lib.EC_ERR_NAN):
            check(rc, "ec_step_batch")
        res = []
        for i in range(self.n_seq):
            if not active[i]:
                res.append(None)
                continue
            o = self._outs[i]
            n = o.n_decoded
            res.append(StepOut(o.status, bool(o.refreshed), o.rows, o.n_cand, bool(o.refresh_next), o.emax,
                               list(o.positions[:n]), list(o.ids[:n]), list(o.entropy[:n]),
                               list(o.maxprob[:n])))
        return res

    def run(self, max_steps: Optional[int] = None, stream=None) -> List[List[Optional[StepOut]]]:
        outs = []
        while not self.done and (max_steps is None or len(outs) < max_steps):
            outs.append(self.step(stream))
        return outs


# ---------------------------------------------------------------------- measurement aid
def ec_timing_enable(on: bool) -> None:
    check(load().ec_timing_enable(1 if on else 0), "ec_timing_enable")


def ec_timing_select(kinds=None) -> None:
    """Record only the named groups (names as in ec_timing_read; None: all groups)."""
    mask = 0xFFFFFFFF if kinds is None else sum(1 << _lib.TIMING_KINDS.index(k) for k in kinds)
    check(load().ec_timing_select(mask), "ec_timing_select")


def ec_timing_read(reset: bool = True) -> dict:
    """Per kernel group: summed event ms, launches, algorithmic flops and bytes."""
    t = _lib.ec_timing()
    t.struct_size = C.sizeof(_lib.ec_timing)
    check(load().ec_timing_read(C.byref(t), 1 if reset else 0), "ec_timing_read")
    return {name: {"ms": t.ms[i], "launches": int(t.launches[i]), "flops": t.flops[i],
                   "bytes": t.bytes[i]}
            for i, name in enumerate(_lib.TIMING_KINDS)}
