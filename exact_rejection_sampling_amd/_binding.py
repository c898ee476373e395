"""ctypes binding of libspec_verify.so.

Argument marshalling only: torch supplies device memory and the current stream; every
step of verification runs in the library's HIP kernels.  There is no fallback path:
if the library is missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_NAME = "libspec_verify.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

SPEC_F32, SPEC_BF16 = 0, 1
REQ_STATUS = {0: "OK", 1: "NONFINITE", 2: "BADTOKEN", 3: "BADUNIFORM", 4: "QZERO",
              5: "RESIDUAL_EMPTY", 6: "BADTREE", 7: "INTERNAL"}

_lib = None
_lock = threading.Lock()

_c_void_p, _c_int, _c_float, _c_size_t = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "spec_abi_version": (_c_int, []),
    "spec_trace_set": (_c_int, [_c_void_p, _c_size_t]),
    "spec_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_req_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_chain_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_greedy_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_tree_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_verify_chain": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                   _c_int, _c_int, _c_int, _c_float,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_chain_static": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                          _c_int, _c_int, _c_int, _c_float,
                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "spec_verify_chain_stop": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                        _c_int, _c_int, _c_int, _c_float,
                                        _c_void_p, _c_int, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_greedy": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                                    _c_void_p]),
    "spec_verify_chain_ex": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                      _c_int, _c_int, _c_int, _c_float, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_greedy_ex": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_greedy_stop": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int,
                                         _c_void_p, _c_int, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_tree": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                  _c_int, _c_int, _c_int, _c_float,
                                  _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_tree_greedy": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_size_t, _c_void_p]),
    "spec_tree_residual_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_verify_tree_residual": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                           _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_float,
                                           _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                           _c_void_p, _c_size_t, _c_void_p]),
}


class SpecOptions(ctypes.Structure):
    """spec_verify_options: stop tokens, budget, finish and target logit processors (device
    pointers, NULL = off)."""
    _fields_ = [("stop_tokens", _c_void_p), ("n_stop", ctypes.c_int32), ("budget", _c_void_p),
                ("finish", _c_void_p), ("bias", _c_void_p), ("allowed", _c_void_p), ("top_k", _c_void_p),
                ("top_p", _c_void_p), ("q_index", _c_void_p), ("q_k", ctypes.c_int32),
                ("lazy_rows", ctypes.c_int32)]


class SpecError(RuntimeError):
    """A host-side error status returned by the library."""


def load_library(path: Optional[str] = None, install: bool = False) -> ctypes.CDLL:
    """Load (once) and return the shared library; raises if it has not been built.

    With a path, that library is loaded instead (for instance the timeline-trace build); with
    install=True it also becomes the one every later call of this module uses."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{LIB_NAME} not found at {p}: build it with "
                "`python -m exact_rejection_sampling_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None or install:
            _lib = lib
        return lib


def _check(code: int) -> None:
    if code != 0:
        msg = load_library().spec_status_string(code).decode()
        raise SpecError(f"libspec_verify status {code}: {msg}")


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"{what} must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, what: str, dtype=None, shape=None, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


_WS_CACHE = {}   # (kind, device index, stream handle) -> (workspace tensor, stream)


def workspace(kind: str, size: int, device: torch.device, stream: torch.cuda.Stream) -> torch.Tensor:
    """A zero-initialised workspace of at least `size` bytes, kept per (kind, device, stream).

    Calls on one stream run in order and leave the workspace zeroed, so it is reused;
    calls on different streams get different workspaces.  After a call reports
    SPEC_REQ_INTERNAL, reset_workspaces() zero-fills them again.
    """
    key = (kind, device.index, stream.cuda_stream)
    ent = _WS_CACHE.get(key)
    ws = None if ent is None else ent[0]
    if ws is None or ws.numel() < size:
        with torch.cuda.stream(stream):
            ws = torch.zeros(max(size, 256) + 256, dtype=torch.uint8, device=device)
        _WS_CACHE[key] = (ws, stream)
    return ws


def reset_workspaces(device=None) -> int:
    """Zero-fills the workspaces this module has cached (all of them, or those on `device`),
    each with a fill on the stream it serves; returns how many were reset.

    A wait between blocks that gives up (status SPEC_REQ_INTERNAL) may leave a published
    word behind.  A chain call repairs its own workspace; a greedy or tree call marks it
    dirty, and every later call on it then reports SPEC_REQ_INTERNAL for all its requests
    until the workspace is zero-filled: this does that for the cached ones (a caller-owned
    workspace_tensor is the caller's to zero).  Not for use during graph capture.
    """
    want = None if device is None else torch.device(device).index
    n = 0
    for (kind, dev_index, _), (ws, stream) in list(_WS_CACHE.items()):
        if want is not None and dev_index != want:
            continue
        with torch.cuda.stream(stream):
            ws.zero_()
        n += 1
    return n


def _aligned_ws(ws: torch.Tensor) -> tuple:
    base = ws.data_ptr()
    off = (-base) % 256
    return ctypes.c_void_p(base + off), ws.numel() - off


class PreparedCall:
    """One library call with its arguments marshalled once.

    Holds the tensors it points into (inputs, outputs, workspace) so their memory stays
    alive, and the stream that was current when it was prepared.  Calling it enqueues the
    same work again on that stream; it re-reads the tensors' *current contents*, so a caller
    may refill the inputs in place between calls.
    """

    __slots__ = ("_fn", "_args", "_keep", "out")

    def __init__(self, fn, args, keep, out):
        self._fn, self._args, self._keep, self.out = fn, args, keep, out

    def __call__(self) -> dict:
        code = self._fn(*self._args)
        if code != 0:
            _check(code)
        return self.out


SPEC_MAX_STOP = 256


def _stop_args(stop_tokens, budget, B, dev):
    """Checks the stop-token list [n] and the budget [B] (int32 GPU tensors, either None)."""
    if stop_tokens is not None:
        _need(stop_tokens, "stop_tokens", dtype=torch.int32, device=dev)
        if stop_tokens.dim() != 1 or stop_tokens.numel() > SPEC_MAX_STOP:
            raise ValueError(f"stop_tokens must be 1-D with at most {SPEC_MAX_STOP} entries")
    if budget is not None:
        _need(budget, "budget", dtype=torch.int32, shape=(B,), device=dev)
    n = 0 if stop_tokens is None else int(stop_tokens.numel())
    return n


def _proc_args(bias, allowed, top_k, top_p, B, R, V, dev):
    """Checks the processor tensors: bias [V] fp32, allowed [B, R, ceil(V/32)] int32/uint32
    bit words, top_k [B] int32, top_p [B] fp32 (each None = off)."""
    if bias is not None:
        _need(bias, "bias", dtype=torch.float32, shape=(V,), device=dev)
    if allowed is not None:
        if allowed.dtype not in (torch.int32, torch.uint32):
            raise TypeError("allowed must be int32 or uint32 bit words")
        _need(allowed, "allowed", shape=(B, R, (V + 31) // 32), device=dev)
    if top_k is not None:
        _need(top_k, "top_k", dtype=torch.int32, shape=(B,), device=dev)
    if top_p is not None:
        _need(top_p, "top_p", dtype=torch.float32, shape=(B,), device=dev)


def _options(stop_tokens, budget, finish, bias=None, allowed=None, top_k=None, top_p=None,
             q_index=None, lazy_rows=0) -> SpecOptions:
    o = SpecOptions()
    o.lazy_rows = int(lazy_rows)
    o.q_index = _ptr(q_index)
    o.q_k = 0 if q_index is None else int(q_index.shape[-1])
    o.stop_tokens = _ptr(stop_tokens)
    o.n_stop = 0 if stop_tokens is None else int(stop_tokens.numel())
    o.budget, o.finish = _ptr(budget), _ptr(finish)
    o.bias, o.allowed, o.top_k, o.top_p = _ptr(bias), _ptr(allowed), _ptr(top_k), _ptr(top_p)
    return o


def _chain_args(target_logits, draft_probs, draft_tokens, uniforms, temperature, with_stats,
                workspace_tensor, out, stop_tokens=None, budget=None, bias=None, allowed=None, top_k=None,
                top_p=None, q_index=None, lazy_rows=0):
    lib = load_library()
    if int(lazy_rows) < 0:
        raise ValueError("lazy_rows must be >= 0")
    _need(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, R, V = target_logits.shape
    G = R - 1
    dev = target_logits.device
    if q_index is None:
        _need(draft_probs, "draft_probs", shape=(B, G, V), device=dev)
    else:
        _need(q_index, "q_index", dtype=torch.int32, device=dev)
        if q_index.dim() != 3 or tuple(q_index.shape[:2]) != (B, G):
            raise ValueError("q_index must be [B, gamma, K]")
        _need(draft_probs, "draft_probs", dtype=torch.float32, shape=tuple(q_index.shape), device=dev)
    _need(draft_tokens, "draft_tokens", dtype=torch.int32, shape=(B, G), device=dev)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, R), device=dev)
    lt, qt = _dtype_code(target_logits, "target_logits"), _dtype_code(draft_probs, "draft_probs")
    if out is None:
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, R, dtype=torch.int32, device=dev),
                   req_status=torch.empty(B, dtype=torch.int32, device=dev))
        if with_stats:
            out["stats"] = torch.empty(B, R, 4, dtype=torch.float32, device=dev)
    stopping = stop_tokens is not None or budget is not None
    n_stop = _stop_args(stop_tokens, budget, B, dev)
    processing = any(t is not None for t in (bias, allowed, top_k, top_p, q_index)) or int(lazy_rows) > 0
    _proc_args(bias, allowed, top_k, top_p, B, R, V, dev)
    if stopping and "finish" not in out:
        out["finish"] = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    need = lib.spec_chain_workspace_bytes(B, G, V)
    if need == 0 and B > 0:
        raise SpecError(f"unsupported sizes B={B} gamma={G} V={V}")
    ws = workspace_tensor if workspace_tensor is not None else workspace("chain", need, dev, stream)
    wp, wn = _aligned_ws(ws)
    head = (_ptr(target_logits), lt, _ptr(draft_probs), qt, _ptr(draft_tokens), _ptr(uniforms),
            B, G, V, ctypes.c_float(float(temperature)))
    keep = (target_logits, draft_probs, draft_tokens, uniforms, ws, stream, stop_tokens, budget, bias, allowed,
            top_k, top_p, q_index)
    if processing:
        opt = _options(stop_tokens, budget, out.get("finish"), bias, allowed, top_k, top_p, q_index, lazy_rows)
        args = head + (ctypes.byref(opt), _ptr(out["accepted_len"]), _ptr(out["out_tokens"]),
                       _ptr(out["req_status"]), _ptr(out.get("stats")), wp, wn, ctypes.c_void_p(stream.cuda_stream))
        return lib.spec_verify_chain_ex, args, keep + (opt,), out
    if not stopping:
        args = head + (_ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["req_status"]),
                       _ptr(out.get("stats")), wp, wn, ctypes.c_void_p(stream.cuda_stream))
        return lib.spec_verify_chain, args, keep, out
    args = head + (_ptr(stop_tokens), n_stop, _ptr(budget),
                   _ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["req_status"]),
                   _ptr(out["finish"]), _ptr(out.get("stats")), wp, wn, ctypes.c_void_p(stream.cuda_stream))
    return lib.spec_verify_chain_stop, args, keep, out


def spec_verify_chain(target_logits: torch.Tensor, draft_probs: torch.Tensor,
                      draft_tokens: torch.Tensor, uniforms: torch.Tensor, temperature: float,
                      *, with_stats: bool = False, workspace_tensor: Optional[torch.Tensor] = None,
                      out: Optional[dict] = None, stop_tokens: Optional[torch.Tensor] = None,
                      budget: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                      allowed: Optional[torch.Tensor] = None, top_k: Optional[torch.Tensor] = None,
                      top_p: Optional[torch.Tensor] = None, q_index: Optional[torch.Tensor] = None,
                      lazy_rows: int = 0) -> dict:
    """Chain verification by rejection sampling (C entry point spec_verify_chain;
    spec_verify_chain_stop when stop_tokens or budget is given; spec_verify_chain_ex when a
    processor is given).

    target_logits [B, gamma+1, V] bf16/fp32; draft_probs [B, gamma, V] fp32/bf16;
    draft_tokens [B, gamma] int32; uniforms [B, gamma+1] fp32; temperature > 0;
    stop_tokens [n] int32 (n <= 256); budget [B] int32 remaining output budgets;
    processors: bias [V] fp32, allowed [B, gamma+1, ceil(V/32)] int32 bit words,
    top_k [B] int32, top_p [B] fp32; sparse draft rows: q_index [B, gamma, K] int32 with
    draft_probs [B, gamma, K] fp32 values (every token not listed has q = 0); lazy_rows k >= 1:
    rows read in groups of k, a group only when every draft before it was accepted.
    Returns {accepted_len [B], out_tokens [B, gamma+1], req_status [B], stats?, finish?}
    (int32 / fp32 GPU tensors, valid once the current stream reaches the call).
    """
    fn, args, _, out = _chain_args(target_logits, draft_probs, draft_tokens, uniforms, temperature,
                                   with_stats, workspace_tensor, out, stop_tokens, budget, bias, allowed,
                                   top_k, top_p, q_index, lazy_rows)
    _check(fn(*args))
    return out


def spec_verify_chain_static(target_logits: torch.Tensor, draft_probs: torch.Tensor,
                             draft_tokens: torch.Tensor, uniforms: torch.Tensor, temperature: float,
                             *, with_stats: bool = False, out: Optional[dict] = None) -> dict:
    """spec_verify_chain without a workspace (C entry point spec_verify_chain_static): the
    library's per-GPU static scratch stands in for it, so nothing is allocated when `out`
    is given.  Same arguments, results and errors as spec_verify_chain's plain form."""
    lib = load_library()
    _need(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, R, V = target_logits.shape
    G = R - 1
    dev = target_logits.device
    _need(draft_probs, "draft_probs", shape=(B, G, V), device=dev)
    _need(draft_tokens, "draft_tokens", dtype=torch.int32, shape=(B, G), device=dev)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, R), device=dev)
    lt, qt = _dtype_code(target_logits, "target_logits"), _dtype_code(draft_probs, "draft_probs")
    if out is None:
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, R, dtype=torch.int32, device=dev),
                   req_status=torch.empty(B, dtype=torch.int32, device=dev))
        if with_stats:
            out["stats"] = torch.empty(B, R, 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = lib.spec_verify_chain_static(_ptr(target_logits), lt, _ptr(draft_probs), qt, _ptr(draft_tokens),
                                        _ptr(uniforms), B, G, V, ctypes.c_float(float(temperature)),
                                        _ptr(out["accepted_len"]), _ptr(out["out_tokens"]),
                                        _ptr(out["req_status"]), _ptr(out.get("stats")),
                                        ctypes.c_void_p(stream.cuda_stream))
    if code != 0:
        _check(code)
    return out


def prepare_chain(target_logits, draft_probs, draft_tokens, uniforms, temperature, *,
                  with_stats=False, workspace_tensor=None, out=None, stop_tokens=None,
                  budget=None, bias=None, allowed=None, top_k=None, top_p=None, q_index=None,
                  lazy_rows=0) -> PreparedCall:
    """spec_verify_chain with its arguments checked and marshalled once (see PreparedCall)."""
    return PreparedCall(*_chain_args(target_logits, draft_probs, draft_tokens, uniforms, temperature,
                                     with_stats, workspace_tensor, out, stop_tokens, budget, bias, allowed,
                                     top_k, top_p, q_index, lazy_rows))


def _greedy_args(target_logits, draft_tokens, workspace_tensor, out, stop_tokens=None, budget=None, bias=None,
                 allowed=None, lazy_rows=0):
    lib = load_library()
    if int(lazy_rows) < 0:
        raise ValueError("lazy_rows must be >= 0")
    _need(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, R, V = target_logits.shape
    G = R - 1
    dev = target_logits.device
    _need(draft_tokens, "draft_tokens", dtype=torch.int32, shape=(B, G), device=dev)
    lt = _dtype_code(target_logits, "target_logits")
    if out is None:
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, R, dtype=torch.int32, device=dev),
                   req_status=torch.empty(B, dtype=torch.int32, device=dev))
    stopping = stop_tokens is not None or budget is not None
    n_stop = _stop_args(stop_tokens, budget, B, dev)
    processing = bias is not None or allowed is not None or int(lazy_rows) > 0
    _proc_args(bias, allowed, None, None, B, R, V, dev)
    if stopping and "finish" not in out:
        out["finish"] = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    need = lib.spec_greedy_workspace_bytes(B, G, V)
    if need == 0 and B > 0:
        raise SpecError(f"unsupported sizes B={B} gamma={G} V={V}")
    ws = workspace_tensor if workspace_tensor is not None else workspace("greedy", need, dev, stream)
    wp, wn = _aligned_ws(ws)
    keep = (target_logits, draft_tokens, ws, stream, stop_tokens, budget, bias, allowed)
    head = (_ptr(target_logits), lt, _ptr(draft_tokens), B, G, V)
    if processing:
        opt = _options(stop_tokens, budget, out.get("finish"), bias, allowed, lazy_rows=lazy_rows)
        args = head + (ctypes.byref(opt), _ptr(out["accepted_len"]), _ptr(out["out_tokens"]),
                       _ptr(out["req_status"]), wp, wn, ctypes.c_void_p(stream.cuda_stream))
        return lib.spec_verify_greedy_ex, args, keep + (opt,), out
    if not stopping:
        args = head + (_ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["req_status"]),
                       wp, wn, ctypes.c_void_p(stream.cuda_stream))
        return lib.spec_verify_greedy, args, keep, out
    args = head + (_ptr(stop_tokens), n_stop, _ptr(budget),
                   _ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["req_status"]),
                   _ptr(out["finish"]), wp, wn, ctypes.c_void_p(stream.cuda_stream))
    return lib.spec_verify_greedy_stop, args, keep, out


def spec_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor, *,
                       workspace_tensor: Optional[torch.Tensor] = None,
                       out: Optional[dict] = None, stop_tokens: Optional[torch.Tensor] = None,
                       budget: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                       allowed: Optional[torch.Tensor] = None, lazy_rows: int = 0) -> dict:
    """Greedy argmax-match verification (C entry point spec_verify_greedy;
    spec_verify_greedy_stop when stop_tokens or budget is given; spec_verify_greedy_ex when
    bias, allowed or lazy_rows is given).

    target_logits [B, gamma+1, V] bf16/fp32; draft_tokens [B, gamma] int32; stop_tokens,
    budget, bias, allowed, lazy_rows as for spec_verify_chain.
    """
    fn, args, _, out = _greedy_args(target_logits, draft_tokens, workspace_tensor, out, stop_tokens, budget, bias,
                                    allowed, lazy_rows)
    _check(fn(*args))
    return out


def prepare_greedy(target_logits, draft_tokens, *, workspace_tensor=None, out=None, stop_tokens=None,
                   budget=None, bias=None, allowed=None, lazy_rows=0) -> PreparedCall:
    """spec_verify_greedy with its arguments checked and marshalled once (see PreparedCall)."""
    return PreparedCall(*_greedy_args(target_logits, draft_tokens, workspace_tensor, out, stop_tokens, budget,
                                      bias, allowed, lazy_rows))


def _tree_args(node_logits, node_tokens, parents, uniforms, temperature, workspace_tensor, out):
    """uniforms None: the greedy walk (spec_verify_tree_greedy; temperature unused)."""
    lib = load_library()
    _need(node_logits, "node_logits")
    if node_logits.dim() != 3:
        raise ValueError("node_logits must be [B, N, V]")
    B, N, V = node_logits.shape
    dev = node_logits.device
    _need(node_tokens, "node_tokens", dtype=torch.int32, shape=(B, N), device=dev)
    _need(parents, "parents", dtype=torch.int32, shape=(B, N), device=dev)
    if uniforms is not None:
        _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, N), device=dev)
    lt = _dtype_code(node_logits, "node_logits")
    if out is None:
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, N, dtype=torch.int32, device=dev),
                   out_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
                   req_status=torch.empty(B, dtype=torch.int32, device=dev))
    stream = torch.cuda.current_stream(dev)
    need = lib.spec_tree_workspace_bytes(B, N, V)
    if need == 0 and B > 0:
        raise SpecError(f"unsupported sizes B={B} N={N} V={V}")
    ws = workspace_tensor if workspace_tensor is not None else workspace("tree", need, dev, stream)
    wp, wn = _aligned_ws(ws)
    keep = (node_logits, node_tokens, parents, uniforms, ws, stream)
    outs = (_ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["out_nodes"]),
            _ptr(out["req_status"]), wp, wn, ctypes.c_void_p(stream.cuda_stream))
    if uniforms is None:
        args = (_ptr(node_logits), lt, _ptr(node_tokens), _ptr(parents), B, N, V) + outs
        return lib.spec_verify_tree_greedy, args, keep, out
    args = (_ptr(node_logits), lt, _ptr(node_tokens), _ptr(parents), _ptr(uniforms),
            B, N, V, ctypes.c_float(float(temperature))) + outs
    return lib.spec_verify_tree, args, keep, out


def spec_verify_tree(node_logits: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor,
                     uniforms: torch.Tensor, temperature: float, *,
                     workspace_tensor: Optional[torch.Tensor] = None,
                     out: Optional[dict] = None) -> dict:
    """Tree verification by target-sample membership (C entry point spec_verify_tree).

    node_logits [B, N, V] bf16/fp32 (row v scores the children of node v); node_tokens,
    parents [B, N] int32 (parents[:, 0] = -1, 0 <= parents[v] < v); uniforms [B, N] fp32.
    Returns {accepted_len [B], out_tokens [B, N], out_nodes [B, N], req_status [B]}.
    """
    fn, args, _, out = _tree_args(node_logits, node_tokens, parents, uniforms, temperature,
                                  workspace_tensor, out)
    _check(fn(*args))
    return out


def prepare_tree(node_logits, node_tokens, parents, uniforms, temperature, *, workspace_tensor=None,
                 out=None) -> PreparedCall:
    """spec_verify_tree with its arguments checked and marshalled once (see PreparedCall)."""
    return PreparedCall(*_tree_args(node_logits, node_tokens, parents, uniforms, temperature,
                                    workspace_tensor, out))


def spec_verify_tree_greedy(node_logits: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor, *,
                            workspace_tensor: Optional[torch.Tensor] = None,
                            out: Optional[dict] = None) -> dict:
    """Greedy tree verification, the temperature-0 membership walk (C entry point
    spec_verify_tree_greedy): the target's argmax (lowest index on ties) in place of its
    sample.  Arguments and outputs as spec_verify_tree, without uniforms or temperature.
    """
    fn, args, _, out = _tree_args(node_logits, node_tokens, parents, None, 0.0, workspace_tensor, out)
    _check(fn(*args))
    return out


def prepare_tree_greedy(node_logits, node_tokens, parents, *, workspace_tensor=None, out=None) -> PreparedCall:
    """spec_verify_tree_greedy with its arguments checked and marshalled once (see PreparedCall)."""
    return PreparedCall(*_tree_args(node_logits, node_tokens, parents, None, 0.0, workspace_tensor, out))


def _tree_residual_args(node_logits, draft_probs, node_tokens, parents, accept_uniforms, draw_uniforms,
                        temperature, workspace_tensor, out):
    lib = load_library()
    _need(node_logits, "node_logits")
    if node_logits.dim() != 3:
        raise ValueError("node_logits must be [B, N, V]")
    B, N, V = node_logits.shape
    dev = node_logits.device
    _need(draft_probs, "draft_probs", shape=(B, N, V), device=dev)
    _need(node_tokens, "node_tokens", dtype=torch.int32, shape=(B, N), device=dev)
    _need(parents, "parents", dtype=torch.int32, shape=(B, N), device=dev)
    _need(accept_uniforms, "accept_uniforms", dtype=torch.float32, shape=(B, N), device=dev)
    _need(draw_uniforms, "draw_uniforms", dtype=torch.float32, shape=(B, N), device=dev)
    lt, qt = _dtype_code(node_logits, "node_logits"), _dtype_code(draft_probs, "draft_probs")
    if out is None:
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, N, dtype=torch.int32, device=dev),
                   out_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
                   req_status=torch.empty(B, dtype=torch.int32, device=dev))
    stream = torch.cuda.current_stream(dev)
    need = lib.spec_tree_residual_workspace_bytes(B, N, V)
    if need == 0 and B > 0:
        raise SpecError(f"unsupported sizes B={B} N={N} V={V}")
    ws = workspace_tensor if workspace_tensor is not None else workspace("tree_residual", need, dev, stream)
    wp, wn = _aligned_ws(ws)
    args = (_ptr(node_logits), lt, _ptr(draft_probs), qt, _ptr(node_tokens), _ptr(parents),
            _ptr(accept_uniforms), _ptr(draw_uniforms), B, N, V, ctypes.c_float(float(temperature)),
            _ptr(out["accepted_len"]), _ptr(out["out_tokens"]), _ptr(out["out_nodes"]),
            _ptr(out["req_status"]), wp, wn, ctypes.c_void_p(stream.cuda_stream))
    keep = (node_logits, draft_probs, node_tokens, parents, accept_uniforms, draw_uniforms, ws, stream)
    return lib.spec_verify_tree_residual, args, keep, out


def spec_verify_tree_residual(node_logits: torch.Tensor, draft_probs: torch.Tensor, node_tokens: torch.Tensor,
                              parents: torch.Tensor, accept_uniforms: torch.Tensor, draw_uniforms: torch.Tensor,
                              temperature: float, *, workspace_tensor: Optional[torch.Tensor] = None,
                              out: Optional[dict] = None) -> dict:
    """Multi-candidate tree verification with residual updates (C entry point
    spec_verify_tree_residual).

    node_logits [B, N, V] bf16/fp32; draft_probs [B, N, V] fp32/bf16 (row c: the distribution
    node c's token was drawn from); node_tokens, parents [B, N] int32; accept_uniforms,
    draw_uniforms [B, N] fp32.  Returns {accepted_len, out_tokens, out_nodes, req_status}.
    """
    fn, args, _, out = _tree_residual_args(node_logits, draft_probs, node_tokens, parents, accept_uniforms,
                                           draw_uniforms, temperature, workspace_tensor, out)
    _check(fn(*args))
    return out


def prepare_tree_residual(node_logits, draft_probs, node_tokens, parents, accept_uniforms, draw_uniforms,
                          temperature, *, workspace_tensor=None, out=None) -> PreparedCall:
    """spec_verify_tree_residual with its arguments checked and marshalled once."""
    return PreparedCall(*_tree_residual_args(node_logits, draft_probs, node_tokens, parents, accept_uniforms,
                                             draw_uniforms, temperature, workspace_tensor, out))


def tree_residual_workspace_bytes(B: int, N: int, V: int) -> int:
    return load_library().spec_tree_residual_workspace_bytes(B, N, V)


def chain_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return load_library().spec_chain_workspace_bytes(B, gamma, V)


def greedy_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return load_library().spec_greedy_workspace_bytes(B, gamma, V)


def tree_workspace_bytes(B: int, N: int, V: int) -> int:
    return load_library().spec_tree_workspace_bytes(B, N, V)
