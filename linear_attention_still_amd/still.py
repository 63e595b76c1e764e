"""ctypes binding of libstill.so (include/still.h), same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers, the
current torch stream as the HIP stream. Every step of the layer runs in the
library's HIP kernels; there is no fallback. A missing or unbuilt library
raises immediately.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstill.so")

STILL_ABI_VERSION = 1
STILL_DTYPE_F32 = 0
STILL_DTYPE_BF16 = 1
STILL_FLAG_FP32_OUT = 1
STILL_FLAG_SOFTMAX_ONLY = 2
STILL_FLAG_MERGE_SUM = 4
STILL_FLAG_PAGED_POOL = 16
STILL_FLAG_POOL_FP8 = 32
STILL_POOL_PAGE_ROWS = 16
# routing metrics (flags bits 8..11)
ROUTES = {"saliency": 0, "diag": 1, "qk": 2, "keynorm": 3, "uniform": 4, "external": 5}


def route_flag(route: str) -> int:
    """The flags bits that select a routing metric (see ROUTES)."""
    return ROUTES[route] << 8
STILL_OK, STILL_EINVAL, STILL_EUNSUPPORTED, STILL_EWORKSPACE, STILL_EHIP, STILL_ESTATE, \
    STILL_ESCRATCH = 0, -1, -2, -3, -4, -5, -6


class still_params(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("budget", ctypes.c_int32), ("t_max", ctypes.c_int32),
                ("eps", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class still_state_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("unit_bytes", "S", "z", "pool_k", "pool_v", "pool_pos", "ring_k", "ring_v",
                 "ring_phi", "ring_flag", "pending", "meta")] + \
               [("ring_slots", ctypes.c_int32), ("pool_slots", ctypes.c_int32)]


class StillError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__("%s failed: %s (%d)" % (fn, still_status_str(rc), rc))
        self.rc = rc


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libstill.so is not built (%s); run __graft_entry__.build() "
                               "or python -m linear_attention_still_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        pp = ctypes.POINTER(still_params)
        L.still_lambda.argtypes = [pp]
        L.still_lambda.restype = I32
        L.still_state_layout_get.argtypes = [pp, ctypes.POINTER(still_state_layout)]
        L.still_state_layout_get.restype = I32
        L.still_state_bytes.argtypes = [pp]
        L.still_state_bytes.restype = I64
        L.still_workspace_bytes.argtypes = [pp, I64]
        L.still_workspace_bytes.restype = I64
        L.still_prefill.argtypes = [pp, I64] + [P] * 10 + [ctypes.c_size_t, P]
        L.still_prefill.restype = I32
        L.still_prefill_gated.argtypes = [pp, I64] + [P] * 11 + [ctypes.c_size_t, P]
        L.still_prefill_gated.restype = I32
        L.still_prefill_decay.argtypes = [pp, I64] + [P] * 11 + [ctypes.c_size_t, P]
        L.still_prefill_decay.restype = I32
        L.still_prefill_paged.argtypes = [pp, I64] + [P] * 11 + [I64, P, ctypes.c_size_t, P]
        L.still_prefill_paged.restype = I32
        L.still_decode_step_paged.argtypes = [pp, I64] + [P] * 8 + [I64, P, P, P]
        L.still_decode_step_paged.restype = I32
        L.still_pool_rows.argtypes = [pp, I64]
        L.still_pool_rows.restype = I64
        L.still_decode_step_gated.argtypes = [pp, I64] + [P] * 10
        L.still_decode_step_gated.restype = I32
        L.still_decode_step_decay.argtypes = [pp, I64] + [P] * 10
        L.still_decode_step_decay.restype = I32
        L.still_prefill_timed.argtypes = [pp, I64] + [P] * 10 + [ctypes.c_size_t, P, P, I32]
        L.still_prefill_timed.restype = I32
        L.still_prefill_partials.argtypes = [pp, I64] + [P] * 10 + [ctypes.c_size_t, P] + [P] * 4
        L.still_prefill_partials.restype = I32
        L.still_prefill_noalloc.argtypes = [pp, I64] + [P] * 10
        L.still_prefill_noalloc.restype = I32
        L.still_noalloc_scratch_bytes.argtypes = []
        L.still_noalloc_scratch_bytes.restype = I64
        L.still_decode_step.argtypes = [pp, I64] + [P] * 9 + [ctypes.c_size_t, P]
        L.still_decode_tokens.argtypes = [pp, I64, P, I32] + [P] * 9
        L.still_decode_tokens.restype = I32
        L.still_workspace_bytes_varlen.argtypes = [pp, P]
        L.still_workspace_bytes_varlen.restype = I64
        L.still_prefill_varlen.argtypes = [pp, P] + [P] * 10 + [ctypes.c_size_t, P]
        L.still_prefill_varlen.restype = I32
        L.still_backward_workspace_bytes.argtypes = [pp, I64]
        L.still_backward_workspace_bytes.restype = I64
        L.still_backward.argtypes = [pp, I64] + [P] * 15 + [P, ctypes.c_size_t, P]
        L.still_backward.restype = I32
        L.still_decode_step.restype = I32
        L.still_status_str.argtypes = [I32]
        L.still_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_params(*, dtype: str, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                window: int, chunk: int, budget: int, t_max: int, eps: float = 0.0,
                sm_scale: float = 0.0, fp32_out: bool = False, flags: int = 0) -> still_params:
    """eps <= 0 and sm_scale <= 0 select the library defaults (1e-6 and
    1/sqrt(head_dim)); flags are further STILL_FLAG_* bits."""
    return still_params(STILL_ABI_VERSION,
                        STILL_DTYPE_F32 if dtype in ("f32", torch.float32) else STILL_DTYPE_BF16,
                        batch, n_q_heads, n_kv_heads, head_dim, window, chunk, budget, t_max,
                        eps, sm_scale, (STILL_FLAG_FP32_OUT if fp32_out else 0) | flags)


def params_for(wl, fp32_out: bool = False, flags: int = 0) -> still_params:
    """Parameters of a Workload (linear_attention_still_amd.inputs)."""
    return make_params(dtype=wl.dtype, batch=wl.batch, n_q_heads=wl.n_q_heads,
                       n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim, window=wl.window,
                       chunk=wl.chunk, budget=wl.budget, t_max=wl.t_max, fp32_out=fp32_out,
                       flags=flags)


def still_status_str(rc: int) -> str:
    return lib().still_status_str(rc).decode()


def still_lambda(p: still_params) -> int:
    rc = lib().still_lambda(ctypes.byref(p))
    if rc < 0:
        raise StillError("still_lambda", rc)
    return rc


def still_state_layout_get(p: still_params) -> still_state_layout:
    out = still_state_layout()
    rc = lib().still_state_layout_get(ctypes.byref(p), ctypes.byref(out))
    if rc != STILL_OK:
        raise StillError("still_state_layout_get", rc)
    return out


def still_state_bytes(p: still_params) -> int:
    n = lib().still_state_bytes(ctypes.byref(p))
    if n < 0:
        raise StillError("still_state_bytes", int(n))
    return int(n)


def still_workspace_bytes(p: still_params, seq_len: int) -> int:
    n = lib().still_workspace_bytes(ctypes.byref(p), int(seq_len))
    if n < 0:
        raise StillError("still_workspace_bytes", int(n))
    return int(n)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libstill must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def still_prefill(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out, sel_idx, score,
                  state, workspace, stream=None) -> None:
    rc = lib().still_prefill(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx), _ptr(score),
                             _ptr(state), _ptr(workspace),
                             workspace.numel() * workspace.element_size() if workspace is not None else 0,
                             _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill", rc)


def still_prefill_gated(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out_gate, out,
                        sel_idx, score, state, workspace, stream=None) -> None:
    rc = lib().still_prefill_gated(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(fmap_w), _ptr(gate), _ptr(out_gate), _ptr(out),
                                   _ptr(sel_idx), _ptr(score), _ptr(state), _ptr(workspace),
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill_gated", rc)


def still_prefill_decay(p: still_params, seq_len: int, q, k, v, fmap_w, gate, decay, out,
                        sel_idx, score, state, workspace, stream=None) -> None:
    rc = lib().still_prefill_decay(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(fmap_w), _ptr(gate), _ptr(decay), _ptr(out),
                                   _ptr(sel_idx), _ptr(score), _ptr(state), _ptr(workspace),
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill_decay", rc)


def still_prefill_paged(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out, sel_idx, score,
                        state, pool_pages, page_table, workspace, stream=None) -> None:
    """pool_pages: [n_pages, 2, STILL_POOL_PAGE_ROWS, d] device tensor of the
    params' dtype; page_table: int32 [B * Hkv, width] (see include/still.h)."""
    rc = lib().still_prefill_paged(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx), _ptr(score),
                                   _ptr(state), _ptr(pool_pages), _ptr(page_table),
                                   int(pool_pages.shape[0]), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill_paged", rc)


def still_pool_rows(p: still_params, n_tokens: int) -> int:
    r = int(lib().still_pool_rows(ctypes.byref(p), int(n_tokens)))
    if r < 0:
        raise StillError("still_pool_rows", r)
    return r


def pool_table_width(p: still_params) -> int:
    return (p.budget - p.window + STILL_POOL_PAGE_ROWS - 1) // STILL_POOL_PAGE_ROWS


def still_prefill_partials(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out, sel_idx,
                           score, state, workspace, y_sa, lse_sa, y_la, lse_la,
                           stream=None) -> None:
    rc = lib().still_prefill_partials(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx),
                                      _ptr(score), _ptr(state), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream), _ptr(y_sa), _ptr(lse_sa), _ptr(y_la),
                                      _ptr(lse_la))
    if rc != STILL_OK:
        raise StillError("still_prefill_partials", rc)


def still_prefill_noalloc(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out, sel_idx,
                          score, state, stream=None) -> None:
    rc = lib().still_prefill_noalloc(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx),
                                     _ptr(score), _ptr(state), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill_noalloc", rc)


def still_noalloc_scratch_bytes() -> int:
    return int(lib().still_noalloc_scratch_bytes())


PREFILL_KERNELS = ("fmap_transpose", "score", "select", "state_delta", "state_scan", "attend",
                   "export")


def still_prefill_timed(p: still_params, seq_len: int, q, k, v, fmap_w, gate, out, sel_idx,
                        score, state, workspace, events, stream=None) -> None:
    """events: flat list of 2*n torch.cuda.Event (enable_timing=True), already
    recorded once so their handles exist, or None (not recorded); kernel i is
    bracketed by events[2i], events[2i+1]."""
    n = len(events) // 2
    arr = (ctypes.c_void_p * (2 * n))(*[ctypes.c_void_p(e.cuda_event if e is not None else None)
                                        for e in events])
    rc = lib().still_prefill_timed(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx),
                                   _ptr(score), _ptr(state), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(stream), arr, n)
    if rc != STILL_OK:
        raise StillError("still_prefill_timed", rc)


def still_decode_step(p: still_params, pos: int, q, k, v, fmap_w, gate, state, out,
                      sel_new=None, workspace=None, stream=None) -> None:
    rc = lib().still_decode_step(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(fmap_w), _ptr(gate), _ptr(state), _ptr(out),
                                 _ptr(sel_new), _ptr(workspace),
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_decode_step", rc)


def still_decode_step_gated(p: still_params, pos: int, q, k, v, fmap_w, gate, out_gate, state,
                            out, sel_new=None, stream=None) -> None:
    rc = lib().still_decode_step_gated(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(fmap_w), _ptr(gate), _ptr(out_gate), _ptr(state),
                                       _ptr(out), _ptr(sel_new), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_decode_step_gated", rc)


def still_decode_step_decay(p: still_params, pos: int, q, k, v, fmap_w, gate, decay, state, out,
                            sel_new=None, stream=None) -> None:
    rc = lib().still_decode_step_decay(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(fmap_w), _ptr(gate), _ptr(decay), _ptr(state),
                                       _ptr(out), _ptr(sel_new), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_decode_step_decay", rc)


def still_decode_step_paged(p: still_params, pos: int, q, k, v, fmap_w, gate, state, pool_pages,
                            page_table, out, sel_new=None, stream=None) -> None:
    rc = lib().still_decode_step_paged(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(fmap_w), _ptr(gate), _ptr(state), _ptr(pool_pages),
                                       _ptr(page_table), int(pool_pages.shape[0]), _ptr(out),
                                       _ptr(sel_new), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_decode_step_paged", rc)


# ---- allocation helpers (torch memory only) --------------------------------

def _lens(seq_lens):
    a = (ctypes.c_int64 * len(seq_lens))(*[int(x) for x in seq_lens])
    return a


def still_workspace_bytes_varlen(p: still_params, seq_lens) -> int:
    if len(seq_lens) != p.batch:
        raise ValueError("one length per batch row")
    n = int(lib().still_workspace_bytes_varlen(ctypes.byref(p), _lens(seq_lens)))
    if n < 0:
        raise StillError("still_workspace_bytes_varlen", n)
    return n


def still_prefill_varlen(p: still_params, seq_lens, q, k, v, fmap_w, gate, out, sel_idx, score,
                         state, workspace, stream=None) -> None:
    """Rows of their own lengths; q, k, v, out, sel_idx and score packed row
    after row (see include/still.h)."""
    if len(seq_lens) != p.batch:
        raise ValueError("one length per batch row")
    rc = lib().still_prefill_varlen(ctypes.byref(p), _lens(seq_lens), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(fmap_w), _ptr(gate), _ptr(out), _ptr(sel_idx),
                                    _ptr(score), _ptr(state), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_prefill_varlen", rc)


def still_decode_tokens(p: still_params, pos: int, row_pos, q, k, v, fmap_w, gate, state, out,
                        sel_new=None, stream=None) -> None:
    """len(q) decode steps; row_pos: None (every row at pos + s) or a device
    int32 tensor [B] of per-row positions of the first token."""
    n = q.shape[0]
    rc = lib().still_decode_tokens(ctypes.byref(p), int(pos), _ptr(row_pos), int(n), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(fmap_w), _ptr(gate), _ptr(state),
                                   _ptr(out), _ptr(sel_new), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_decode_tokens", rc)


def still_backward_workspace_bytes(p: still_params, seq_len: int) -> int:
    n = int(lib().still_backward_workspace_bytes(ctypes.byref(p), int(seq_len)))
    if n < 0:
        raise StillError("still_backward_workspace_bytes", n)
    return n


def still_backward(p: still_params, seq_len: int, q, k, v, fmap_w, gate, sel_idx, y, lse_sa,
                   lse_la, dy, dq, dk, dv, dfmap, dgate, workspace, stream=None) -> None:
    """Gradients of sum(y * dy), the routing held fixed (see include/still.h)."""
    rc = lib().still_backward(ctypes.byref(p), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(fmap_w), _ptr(gate), _ptr(sel_idx), _ptr(y), _ptr(lse_sa),
                              _ptr(lse_la), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dfmap),
                              _ptr(dgate), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != STILL_OK:
        raise StillError("still_backward", rc)


class PrefillBuffers:
    """Device buffers of one prefill: outputs, kept indices, scores, state,
    workspace."""

    def __init__(self, p: still_params, seq_len: int, device="cuda", fp32_out=None):
        B, Hq, Hkv, d = p.batch, p.n_q_heads, p.n_kv_heads, p.head_dim
        lam = still_lambda(p)
        n_dec = (seq_len - 1) // p.chunk
        fp32 = (p.flags & STILL_FLAG_FP32_OUT) if fp32_out is None else fp32_out
        odt = torch.float32 if (fp32 or p.dtype == STILL_DTYPE_F32) else torch.bfloat16
        self.out = torch.empty((B, Hq, seq_len, d), dtype=odt, device=device)
        self.sel = torch.empty((B, Hkv, n_dec, lam), dtype=torch.int32, device=device)
        self.score = torch.empty((B, Hkv, seq_len), dtype=torch.float32, device=device)
        self.state = torch.zeros((still_state_bytes(p),), dtype=torch.uint8, device=device)
        self.workspace = torch.empty((still_workspace_bytes(p, seq_len),), dtype=torch.uint8,
                                     device=device)


def run_prefill(p: still_params, x: dict, bufs: PrefillBuffers, stream=None) -> PrefillBuffers:
    L = x["q"].shape[2]
    still_prefill(p, L, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], bufs.out,
                  bufs.sel if bufs.sel.numel() else None, bufs.score, bufs.state,
                  bufs.workspace, stream)
    return bufs


def state_views(p: still_params, state: torch.Tensor) -> dict:
    """Typed views of the state blob, per unit (batch row, kv head)."""
    lay = still_state_layout_get(p)
    U = p.batch * p.n_kv_heads
    d, R, P, C = p.head_dim, lay.ring_slots, lay.pool_slots, p.chunk
    edt = torch.float32 if p.dtype == STILL_DTYPE_F32 else torch.bfloat16
    es = 4 if p.dtype == STILL_DTYPE_F32 else 2
    blob = state.view(U, lay.unit_bytes)

    def sec(off, n, dt, size):
        return blob[:, off:off + n * size].contiguous().view(dt).view(U, n)
    if p.flags & STILL_FLAG_POOL_FP8:  # E4M3 codes, then one exponent byte (+127) per row
        extra = {"pool_k8": sec(lay.pool_k, P * d, torch.uint8, 1).view(U, P, d),
                 "pool_k_exp": sec(lay.pool_k + P * d, P, torch.uint8, 1),
                 "pool_v8": sec(lay.pool_v, P * d, torch.uint8, 1).view(U, P, d),
                 "pool_v_exp": sec(lay.pool_v + P * d, P, torch.uint8, 1)}
        edt_pool = None
    else:
        extra, edt_pool = {}, edt
    return {**extra,
        "S": sec(lay.S, d * d, torch.float32, 4).view(U, d, d),
        "z": sec(lay.z, d, torch.float32, 4),
        # (a paged pool keeps its rows in the caller's pages: empty here)
        "pool_k": sec(lay.pool_k, P * d, edt, es).view(U, P, d)
        if edt_pool is not None and not p.flags & STILL_FLAG_PAGED_POOL else None,
        "pool_v": sec(lay.pool_v, P * d, edt, es).view(U, P, d)
        if edt_pool is not None and not p.flags & STILL_FLAG_PAGED_POOL else None,
        "pool_pos": sec(lay.pool_pos, P, torch.int32, 4),
        "ring_k": sec(lay.ring_k, R * d, edt, es).view(U, R, d),
        "ring_v": sec(lay.ring_v, R * d, edt, es).view(U, R, d),
        "ring_phi": sec(lay.ring_phi, R * d, edt, es).view(U, R, d),
        "ring_flag": sec(lay.ring_flag, R, torch.int32, 4),
        "pending": sec(lay.pending, C, torch.float64, 8),
        "meta": sec(lay.meta, 4, torch.int64, 8),
    }


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
