"""ctypes binding of ``libspecdec.so`` (the C ABI in ``include/specdec.h``).

Argument marshalling only: torch device tensors are checked for device, dtype, contiguity and
shape, turned into raw pointers and handed to the library together with the current HIP
stream.  Every step of the verify computation runs in the library's HIP kernels; there is no
CPU or PyTorch fallback, and a missing library raises ``SpecdecError``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import pathlib

import numpy as np
import torch

_LIB = None

SPECDEC_F32 = 0
SPECDEC_BF16 = 1
SPECDEC_MAX_K = 63


class SpecdecError(RuntimeError):
    pass


class _Options(ctypes.Structure):
    _fields_ = [("hot_event_begin", ctypes.c_void_p), ("hot_event_end", ctypes.c_void_p),
                ("path", ctypes.c_int32), ("spin_limit", ctypes.c_int32),
                ("draw_event_begin", ctypes.c_void_p), ("draw_event_end", ctypes.c_void_p)]


# Execution paths of specdec_verify (include/specdec.h).
SPECDEC_SMALL_V_MAX = 1024
SPECDEC_PATH_AUTO, SPECDEC_PATH_STREAMING, SPECDEC_PATH_SMALL_VOCAB = 0, 1, 2
SPECDEC_PATH_ONE_LAUNCH = 3
SPECDEC_PATH_QUAD = 4


def _event_pair(events):
    return (None, None) if events is None else tuple(
        e if isinstance(e, int) or e is None else e.cuda_event for e in events)


def _options(hot_events, path, spin_limit=0, draw_events=None):
    ev, dv = _event_pair(hot_events), _event_pair(draw_events)
    return _Options(ev[0], ev[1], int(path), int(spin_limit), dv[0], dv[1])


def library_path() -> pathlib.Path:
    env = os.environ.get("SPECDEC_LIBRARY")
    return pathlib.Path(env) if env else pathlib.Path(__file__).with_name("libspecdec.so")


def load_library():
    """Load the HIP library once; raise SpecdecError if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not path.exists():
        raise SpecdecError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                           f"g.build()'` (hipcc, gfx950). There is no fallback path.")
    lib = ctypes.CDLL(str(path))
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    common = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.specdec_verify.argtypes = common
    lib.specdec_verify.restype = i32
    lib.specdec_verify_ex.argtypes = common + [ctypes.POINTER(_Options)]
    lib.specdec_verify_ex.restype = i32
    lib.specdec_verify_greedy.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.specdec_verify_greedy.restype = i32
    lib.specdec_verify_match.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp,
                                         sz, vp]
    lib.specdec_verify_match.restype = i32
    lib.specdec_verify_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp,
                                           vp, vp]
    lib.specdec_verify_noalloc.restype = i32
    lib.specdec_noalloc_scratch_bytes.argtypes = []
    lib.specdec_noalloc_scratch_bytes.restype = sz
    lib.specdec_workspace_size.argtypes = [i32, i32, i32]
    lib.specdec_workspace_size.restype = sz
    lib.specdec_ngram_workspace_size.argtypes = [i32, i32]
    lib.specdec_ngram_workspace_size.restype = sz
    lib.specdec_ngram_propose.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.specdec_ngram_propose.restype = i32
    lib.specdec_commit.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.specdec_commit.restype = i32
    lib.specdec_telemetry_update.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    lib.specdec_telemetry_update.restype = i32
    lib.specdec_apply_k.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.specdec_apply_k.restype = i32
    f64 = ctypes.c_double
    lib.specdec_alpha_estimate.argtypes = [vp]
    lib.specdec_alpha_estimate.restype = f64
    lib.specdec_expected_tokens.argtypes = [f64, i32]
    lib.specdec_expected_tokens.restype = f64
    lib.specdec_speedup.argtypes = [f64, i32, f64]
    lib.specdec_speedup.restype = f64
    lib.specdec_choose_k.argtypes = [f64, f64, i32, i32]
    lib.specdec_choose_k.restype = i32
    lib.specdec_plan_k.argtypes = [vp, i32, f64, i32, i32, i32, vp]
    lib.specdec_plan_k.restype = i32
    lib.specdec_status_string.argtypes = [i32]
    lib.specdec_status_string.restype = ctypes.c_char_p
    lib.specdec_version.argtypes = []
    lib.specdec_version.restype = i32
    _LIB = lib
    return lib


def specdec_status_string(status: int) -> str:
    return load_library().specdec_status_string(int(status)).decode()


def specdec_workspace_size(B: int, K: int, V: int) -> int:
    return int(load_library().specdec_workspace_size(int(B), int(K), int(V)))


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor | None, name: str, dtype, shape, device, optional=False):
    if t is None:
        if optional:
            return
        raise SpecdecError(f"{name} is required")
    if t.device != device:
        raise SpecdecError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise SpecdecError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise SpecdecError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise SpecdecError(f"{name} must be contiguous")


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _on(stream):
    """Allocation context for buffers a call creates itself: they belong to the stream the call
    is enqueued on, so torch's caching allocator does not hand them to other work on its current
    stream while the library's kernels still use them."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _outputs(B, K, device, out, want_probs, stream=None):
    if out is not None:
        return out
    with _on(stream):
        acc = torch.empty(B, dtype=torch.int32, device=device)
        tok = torch.empty((B, K + 1), dtype=torch.int32, device=device)
        prb = (torch.empty((B, K + 1), dtype=torch.float32, device=device) if want_probs
               else None)
    return acc, tok, prb


def new_workspace(B: int, K: int, V: int, device, stream=None) -> torch.Tensor:
    """A verify workspace for these sizes (uninitialised: the library needs none), allocated
    for ``stream``."""
    need = specdec_workspace_size(B, K, V)
    with _on(stream):
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def _workspace(B, K, V, device, workspace, stream=None):
    need = specdec_workspace_size(B, K, V)
    if workspace is None:
        workspace = new_workspace(B, K, V, device, stream)
    return workspace, need


def _raise(status: int, fn: str):
    if status != 0:
        raise SpecdecError(f"{fn}: {specdec_status_string(status)} (status {status})")


def specdec_verify(target_logits: torch.Tensor, draft_probs: torch.Tensor | None,
                   proposed: torch.Tensor | None, temperature: torch.Tensor,
                   uniforms: torch.Tensor, *, draft_onehot: torch.Tensor | None = None,
                   num_draft: torch.Tensor | None = None, out=None, workspace=None,
                   want_probs: bool = True, stream=None, hot_events=None,
                   path: int = SPECDEC_PATH_AUTO, spin_limit: int = 0, draw_events=None):
    """Batched verify.  Shapes: target_logits [B, K+1, V] (bf16 or fp32), draft_probs
    [B, K, V] fp32 or None, proposed [B, K] int32, temperature [B] fp32, uniforms [B, K+1]
    fp32, draft_onehot [B] uint8 or None, num_draft [B] int32 or None.  Returns
    (accept_len [B] int32, out_tokens [B, K+1] int32, out_probs [B, K+1] fp32 or None),
    enqueued on ``stream`` (default: torch's current stream) without synchronising.
    ``hot_events``: optional (begin, end) pair of hipEvent_t handles (ints) recorded around the
    kernel that reads every target row; ``draw_events`` the same around the kernels after it
    (streaming path only).  ``path``: SPECDEC_PATH_AUTO (the one-kernel small-vocabulary
    path when V <= SPECDEC_SMALL_V_MAX, else the streaming kernels), _STREAMING, _SMALL_VOCAB
    or _ONE_LAUNCH.
    ``workspace``: a uint8 tensor of at least specdec_workspace_size(B, K, V) bytes
    (``new_workspace``), reusable across calls; None allocates one for this call.
    ``spin_limit``: SPECDEC_PATH_ONE_LAUNCH only, polls of a bounded wait (0 = the default)."""
    lib = load_library()
    if target_logits.dim() != 3:
        raise SpecdecError("target_logits must be [B, K+1, V]")
    B, K1, V = (int(s) for s in target_logits.shape)
    K = K1 - 1
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = SPECDEC_BF16
    elif target_logits.dtype == torch.float32:
        dt = SPECDEC_F32
    else:
        raise SpecdecError(f"target_logits dtype {target_logits.dtype} is not bf16/fp32")
    if not target_logits.is_contiguous():
        raise SpecdecError("target_logits must be contiguous")
    _check(draft_probs, "draft_probs", torch.float32, (B, K, V), dev, optional=True)
    _check(proposed, "proposed", torch.int32, (B, K), dev, optional=(K == 0))
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _check(draft_onehot, "draft_onehot", torch.uint8, (B,), dev, optional=True)
    _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
    acc, tok, prb = _outputs(B, K, dev, out, want_probs, stream)
    ws, need = _workspace(B, K, V, dev, workspace, stream)
    args = (_ptr(target_logits), dt, _ptr(draft_probs), _ptr(draft_onehot), _ptr(proposed),
            _ptr(num_draft), _ptr(temperature), _ptr(uniforms), B, K, V, _ptr(acc), _ptr(tok),
            _ptr(prb), _ptr(ws), ws.numel(), _stream_handle(stream))
    if (hot_events is None and draw_events is None and path == SPECDEC_PATH_AUTO
            and spin_limit == 0):
        status = lib.specdec_verify(*args)
    else:
        opts = _options(hot_events, path, spin_limit, draw_events)
        status = lib.specdec_verify_ex(*args, ctypes.byref(opts))
    _raise(status, "specdec_verify")
    return acc, tok, prb


def specdec_verify_noalloc(target_logits: torch.Tensor, draft_probs: torch.Tensor | None,
                           proposed: torch.Tensor | None, temperature: torch.Tensor,
                           uniforms: torch.Tensor, *, draft_onehot: torch.Tensor | None = None,
                           num_draft: torch.Tensor | None = None, out, stream=None):
    """specdec_verify through the entry point that allocates nothing: its workspace is the
    library's built-in device scratch (``out`` = (accept_len, out_tokens, out_probs or None) is
    required, so that this call creates no tensor either).  Shapes as for specdec_verify."""
    lib = load_library()
    if target_logits.dim() != 3:
        raise SpecdecError("target_logits must be [B, K+1, V]")
    B, K1, V = (int(s) for s in target_logits.shape)
    K = K1 - 1
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = SPECDEC_BF16
    elif target_logits.dtype == torch.float32:
        dt = SPECDEC_F32
    else:
        raise SpecdecError(f"target_logits dtype {target_logits.dtype} is not bf16/fp32")
    if not target_logits.is_contiguous():
        raise SpecdecError("target_logits must be contiguous")
    _check(draft_probs, "draft_probs", torch.float32, (B, K, V), dev, optional=True)
    _check(proposed, "proposed", torch.int32, (B, K), dev, optional=(K == 0))
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _check(draft_onehot, "draft_onehot", torch.uint8, (B,), dev, optional=True)
    _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
    acc, tok, prb = out
    _check(acc, "accept_len", torch.int32, (B,), dev)
    _check(tok, "out_tokens", torch.int32, (B, K + 1), dev)
    _check(prb, "out_probs", torch.float32, (B, K + 1), dev, optional=True)
    status = lib.specdec_verify_noalloc(_ptr(target_logits), dt, _ptr(draft_probs),
                                        _ptr(draft_onehot), _ptr(proposed), _ptr(num_draft),
                                        _ptr(temperature), _ptr(uniforms), B, K, V, _ptr(acc),
                                        _ptr(tok), _ptr(prb), _stream_handle(stream))
    _raise(status, "specdec_verify_noalloc")
    return acc, tok, prb


def specdec_verify_greedy(target_logits: torch.Tensor, proposed: torch.Tensor | None, *,
                          num_draft: torch.Tensor | None = None, out=None, workspace=None,
                          want_probs: bool = True, stream=None):
    """Greedy-only verify (every row at temperature 0).  Returns (accept_len, out_tokens,
    out_probs or None)."""
    lib = load_library()
    if target_logits.dim() != 3:
        raise SpecdecError("target_logits must be [B, K+1, V]")
    B, K1, V = (int(s) for s in target_logits.shape)
    K = K1 - 1
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = SPECDEC_BF16
    elif target_logits.dtype == torch.float32:
        dt = SPECDEC_F32
    else:
        raise SpecdecError(f"target_logits dtype {target_logits.dtype} is not bf16/fp32")
    if not target_logits.is_contiguous():
        raise SpecdecError("target_logits must be contiguous")
    _check(proposed, "proposed", torch.int32, (B, K), dev, optional=(K == 0))
    _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
    acc, tok, prb = _outputs(B, K, dev, out, want_probs, stream)
    ws, need = _workspace(B, K, V, dev, workspace, stream)
    status = lib.specdec_verify_greedy(_ptr(target_logits), dt, _ptr(proposed), _ptr(num_draft),
                                       B, K, V, _ptr(acc), _ptr(tok), _ptr(prb), _ptr(ws),
                                       ws.numel(), _stream_handle(stream))
    _raise(status, "specdec_verify_greedy")
    return acc, tok, prb


def specdec_verify_match(target_logits: torch.Tensor, proposed: torch.Tensor | None,
                         temperature: torch.Tensor, uniforms: torch.Tensor, *,
                         num_draft: torch.Tensor | None = None, out=None, workspace=None,
                         want_probs: bool = True, stream=None):
    """Sample-and-match verify (no draft distribution).  Shapes as for specdec_verify.  Returns
    (accept_len, out_tokens, out_probs or None)."""
    lib = load_library()
    if target_logits.dim() != 3:
        raise SpecdecError("target_logits must be [B, K+1, V]")
    B, K1, V = (int(s) for s in target_logits.shape)
    K = K1 - 1
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = SPECDEC_BF16
    elif target_logits.dtype == torch.float32:
        dt = SPECDEC_F32
    else:
        raise SpecdecError(f"target_logits dtype {target_logits.dtype} is not bf16/fp32")
    if not target_logits.is_contiguous():
        raise SpecdecError("target_logits must be contiguous")
    _check(proposed, "proposed", torch.int32, (B, K), dev, optional=(K == 0))
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
    acc, tok, prb = _outputs(B, K, dev, out, want_probs, stream)
    ws, need = _workspace(B, K, V, dev, workspace, stream)
    status = lib.specdec_verify_match(_ptr(target_logits), dt, _ptr(proposed), _ptr(num_draft),
                                      _ptr(temperature), _ptr(uniforms), B, K, V, _ptr(acc),
                                      _ptr(tok), _ptr(prb), _ptr(ws), ws.numel(),
                                      _stream_handle(stream))
    _raise(status, "specdec_verify_match")
    return acc, tok, prb


def specdec_ngram_workspace_size(B: int, capacity: int) -> int:
    return int(load_library().specdec_ngram_workspace_size(int(B), int(capacity)))


def specdec_ngram_propose(tokens: torch.Tensor, lengths: torch.Tensor, K: int, *, n_min: int = 1,
                          n_max: int = 4, out=None, workspace=None, stream=None):
    """N-gram drafter.  tokens [B, capacity] int32 histories, lengths [B] int32.  Returns
    (proposed [B, K] int32, num_draft [B] int32), enqueued on ``stream`` without synchronising."""
    lib = load_library()
    if tokens.dim() != 2:
        raise SpecdecError("tokens must be [B, capacity]")
    B, cap = (int(s) for s in tokens.shape)
    dev = tokens.device
    _check(tokens, "tokens", torch.int32, (B, cap), dev)
    _check(lengths, "lengths", torch.int32, (B,), dev)
    if out is None:
        with _on(stream):
            out = (torch.empty((B, K), dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev))
    proposed, num_draft = out
    _check(proposed, "proposed", torch.int32, (B, K), dev)
    _check(num_draft, "num_draft", torch.int32, (B,), dev)
    need = specdec_ngram_workspace_size(B, cap)
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    status = lib.specdec_ngram_propose(_ptr(tokens), _ptr(lengths), B, cap, int(n_min), int(n_max),
                                       int(K), _ptr(proposed) if K > 0 else None, _ptr(num_draft),
                                       _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _raise(status, "specdec_ngram_propose")
    return proposed, num_draft


def specdec_commit(accept_len: torch.Tensor, out_tokens: torch.Tensor, seq_len: torch.Tensor, *,
                   tokens: torch.Tensor | None = None, capacity: int | None = None,
                   target_kv_len: torch.Tensor | None = None,
                   draft_kv_len: torch.Tensor | None = None, packed: bool = True, out=None,
                   stream=None):
    """Commit a verified round in place: append the emitted tokens to ``tokens`` [B, capacity]
    (optional), advance ``seq_len`` [B], roll ``target_kv_len`` / ``draft_kv_len`` [B] back
    (optional), and with ``packed`` return (packed_tokens [B*(K+1)], packed_offsets [B+1]);
    otherwise return None.  ``capacity`` defaults to tokens.shape[1]."""
    lib = load_library()
    if out_tokens.dim() != 2:
        raise SpecdecError("out_tokens must be [B, K+1]")
    B, K1 = (int(s) for s in out_tokens.shape)
    dev = out_tokens.device
    _check(accept_len, "accept_len", torch.int32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, K1), dev)
    _check(seq_len, "seq_len", torch.int32, (B,), dev)
    if tokens is not None:
        if tokens.dim() != 2:
            raise SpecdecError("tokens must be [B, capacity]")
        _check(tokens, "tokens", torch.int32, (B, int(tokens.shape[1])), dev)
        cap = int(tokens.shape[1])
        if capacity is not None and int(capacity) != cap:
            raise SpecdecError("capacity differs from tokens.shape[1]")
    elif capacity is None:
        raise SpecdecError("capacity is required when no history tensor is given")
    else:
        cap = int(capacity)
    _check(target_kv_len, "target_kv_len", torch.int32, (B,), dev, optional=True)
    _check(draft_kv_len, "draft_kv_len", torch.int32, (B,), dev, optional=True)
    pk = off = None
    if packed:
        if out is None:
            with _on(stream):
                out = (torch.empty(max(B * K1, 1), dtype=torch.int32, device=dev),
                       torch.empty(B + 1, dtype=torch.int32, device=dev))
        pk, off = out
    status = lib.specdec_commit(_ptr(accept_len), _ptr(out_tokens), B, K1 - 1, _ptr(tokens), cap,
                                _ptr(seq_len), _ptr(target_kv_len), _ptr(draft_kv_len), _ptr(pk),
                                _ptr(off), _stream_handle(stream))
    _raise(status, "specdec_commit")
    return (pk, off) if packed else None


TELEMETRY_ROW = 72
TELEMETRY_MAX_ROUTES = 64


def telemetry_counters(n_routes: int, device) -> torch.Tensor:
    """Zeroed device counters [n_routes, 72] int64 for specdec_telemetry_update."""
    return torch.zeros((n_routes, TELEMETRY_ROW), dtype=torch.int64, device=device)


def specdec_telemetry_update(counters: torch.Tensor, accept_len: torch.Tensor, *,
                             num_draft: torch.Tensor | None = None,
                             route: torch.Tensor | None = None, K: int, stream=None):
    """Add one verified batch to the device counters [n_routes, 72] int64 (in place)."""
    lib = load_library()
    B = int(accept_len.shape[0])
    dev = accept_len.device
    n_routes = int(counters.shape[0])
    _check(counters, "counters", torch.int64, (n_routes, TELEMETRY_ROW), dev)
    _check(accept_len, "accept_len", torch.int32, (B,), dev)
    _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
    _check(route, "route", torch.int32, (B,), dev, optional=True)
    status = lib.specdec_telemetry_update(_ptr(accept_len), _ptr(num_draft), _ptr(route), B,
                                          int(K), n_routes, _ptr(counters), _stream_handle(stream))
    _raise(status, "specdec_telemetry_update")
    return counters


def specdec_apply_k(num_draft: torch.Tensor, k_table: torch.Tensor, *,
                    route: torch.Tensor | None = None, stream=None):
    """Clamp num_draft [B] (in place) to k_table [n_routes] of each sequence's route."""
    lib = load_library()
    B = int(num_draft.shape[0])
    dev = num_draft.device
    _check(num_draft, "num_draft", torch.int32, (B,), dev)
    _check(k_table, "k_table", torch.int32, (int(k_table.shape[0]),), dev)
    _check(route, "route", torch.int32, (B,), dev, optional=True)
    status = lib.specdec_apply_k(_ptr(num_draft), _ptr(route), _ptr(k_table), B,
                                 int(k_table.shape[0]), _stream_handle(stream))
    _raise(status, "specdec_apply_k")
    return num_draft


def specdec_plan_k(counters_host, c: float, k_min: int, k_max: int, k_default: int):
    """Host planner: counters (host int64 [n_routes, 72], numpy or CPU tensor) -> k per route
    (numpy int32), through the library's host arithmetic."""
    import numpy as np
    cnt = np.ascontiguousarray(np.asarray(counters_host, dtype=np.int64))
    n_routes = cnt.shape[0]
    out = np.empty(n_routes, dtype=np.int32)
    status = load_library().specdec_plan_k(cnt.ctypes.data, n_routes, float(c), int(k_min),
                                           int(k_max), int(k_default), out.ctypes.data)
    _raise(status, "specdec_plan_k")
    return out


def inputs_to_device(inp, device) -> dict:
    """Copy a host ``VerifyInputs`` batch to device tensors (bf16 bit patterns become bf16)."""
    def dev(a, dtype=None):
        if a is None:
            return None
        if not a.flags.writeable:  # e.g. a broadcast view: torch wants a writable buffer
            a = np.array(a)
        t = torch.from_numpy(a)
        if dtype is not None:
            t = t.view(dtype)
        return t.to(device).contiguous()
    if inp.logits_dtype == "bf16":
        logits = dev(inp.logits.view("int16"), torch.bfloat16)
    elif inp.logits_dtype == "f32":
        logits = dev(inp.logits)
    else:
        raise SpecdecError(f"logits dtype {inp.logits_dtype!r} has no device form")
    return dict(logits=logits, draft_probs=dev(inp.draft_probs), draft_onehot=dev(inp.draft_onehot),
                proposed=dev(inp.proposed), num_draft=dev(inp.num_draft),
                temperature=dev(inp.temperature), uniforms=dev(inp.uniforms))


class PreparedVerify:
    """A specdec_verify call with its arguments marshalled once (for tight loops and HIP-graph
    capture).  ``__call__(stream=None, hot_events=None, draw_events=None)`` enqueues it on ``stream`` (default:
    torch's current stream) and raises on a non-zero status."""

    def __init__(self, target_logits, draft_probs, proposed, temperature, uniforms, *,
                 draft_onehot=None, num_draft=None, out=None, workspace=None,
                 path=SPECDEC_PATH_AUTO):
        # Validate once through the checked entry point's rules.
        B, K1, V = (int(s) for s in target_logits.shape)
        dev = target_logits.device
        self.lib = load_library()
        self.keep = (target_logits, draft_probs, proposed, temperature, uniforms, draft_onehot,
                     num_draft)
        dt = SPECDEC_BF16 if target_logits.dtype == torch.bfloat16 else SPECDEC_F32
        _check(draft_probs, "draft_probs", torch.float32, (B, K1 - 1, V), dev, optional=True)
        _check(proposed, "proposed", torch.int32, (B, K1 - 1), dev, optional=(K1 == 1))
        _check(temperature, "temperature", torch.float32, (B,), dev)
        _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
        _check(draft_onehot, "draft_onehot", torch.uint8, (B,), dev, optional=True)
        _check(num_draft, "num_draft", torch.int32, (B,), dev, optional=True)
        self.out = _outputs(B, K1 - 1, dev, out, True)
        self.ws, _ = _workspace(B, K1 - 1, V, dev, workspace)
        acc, tok, prb = self.out
        self.path = int(path)
        self.args = (_ptr(target_logits), dt, _ptr(draft_probs), _ptr(draft_onehot),
                     _ptr(proposed), _ptr(num_draft), _ptr(temperature), _ptr(uniforms), B,
                     K1 - 1, V, _ptr(acc), _ptr(tok), _ptr(prb), _ptr(self.ws), self.ws.numel())

    def __call__(self, stream=None, hot_events=None, draw_events=None):
        s = _stream_handle(stream)
        if hot_events is None and draw_events is None and self.path == SPECDEC_PATH_AUTO:
            status = self.lib.specdec_verify(*self.args, s)
        else:
            opts = _options(hot_events, self.path, 0, draw_events)
            status = self.lib.specdec_verify_ex(*self.args, s, ctypes.byref(opts))
        if status != 0:
            _raise(status, "specdec_verify")
        return self.out
