"""Python binding of libqsa (one QSA layer on gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/qsa.h.  Tensors are torch CUDA (HIP) tensors used for
device memory; the stream is torch's current stream unless one is passed.
There is no fallback: if the library is not built, or a call is rejected,
a QSAError is raised.

Function names follow the C ABI: rope_apply, compress_block_keys,
index_scores, select_topk, sparse_attn_prefill, sparse_attn_decode.  Two
helpers chain them for a whole prefill chunk or decode step.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# QSA_LIBRARY names another build of the same library (the host-sanitizer
# build of block_sparse_long_12_amd.build_sanitize); default: the in-tree one.
LIB_PATH = os.environ.get("QSA_LIBRARY") or os.path.join(HERE, "libqsa.so")

BLOCK, HQ, HKV, D, ROT, HI, DI = 4, 24, 2, 256, 64, 4, 128
ROPE_THETA = 1.0e7
MAX_BATCH = 256
MAX_BUDGET = 2048
NOALLOC_SCRATCH_BYTES = 16 << 20      # QSA_NOALLOC_SCRATCH_BYTES: the static scratch of decode_step_noalloc

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class Rope(ctypes.Structure):
    """Rotary parameters (qsa_rope_t): theta, and static YaRN with scale factor
    yarn_factor over yarn_original_max positions (yarn_factor 1: plain rotary)."""
    _fields_ = [("theta", ctypes.c_double), ("yarn_factor", ctypes.c_double), ("yarn_original_max", ctypes.c_int64)]


def rope_params(theta: float = ROPE_THETA, yarn_factor: float = 1.0, yarn_original_max: int = 0) -> Rope:
    return Rope(float(theta), float(yarn_factor), int(yarn_original_max))


# model card, "Processing Ultra-Long Texts": static YaRN for contexts past 262144
YARN = rope_params(ROPE_THETA, 4.0, 262144)
_rope_p = ctypes.POINTER(Rope)


class _PagedCacheC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_idx", ctypes.c_void_p),
                ("kbar", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
                ("page_tokens", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_paged_p = ctypes.POINTER(_PagedCacheC)


def _rope_arg(rope: Rope | None):
    if rope is None:
        return None
    if not isinstance(rope, Rope):
        raise QSAError("rope must be a qsa.Rope (see rope_params)")
    return ctypes.byref(rope)

_SIGNATURES = {
    "qsa_abi_version": (_i32, []),
    "qsa_get_dims": (_i32, [_c_p]),
    "qsa_status_string": (ctypes.c_char_p, [_i32]),
    "qsa_last_error": (ctypes.c_char_p, []),
    "qsa_rope_apply": (_i32, [_c_p, _i64, _i64, _c_p, _i64, _i64, _i32, _i32, _i32, _c_p,
                              _rope_p, _c_p]),
    "qsa_compress_block_keys": (_i32, [_c_p, _i64, _i32, _i32, _i32, _c_p, _i64, _c_p]),
    "qsa_index_scores": (_i32, [_c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _c_p, _i64, _i64, _c_p]),
    "qsa_select_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "qsa_select_topk": (_i32, [_c_p, _i64, _i64, _c_p, _i32, _i32, _i32, _c_p, _i64, _c_p, _sz, _c_p]),
    "qsa_index_select_prefill_workspace_bytes": (_sz, [_i32, _i32]),
    "qsa_index_select_prefill": (_i32, [_c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _i32, _c_p, _i64, _i64,
                                        _c_p, _i64, _c_p, _sz, _c_p]),
    "qsa_sparse_attn_prefill": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _i32, _i32,
                                       _i32, ctypes.c_float, _c_p, _i64, _c_p, _i64, _c_p, _i64, _c_p]),
    "qsa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "qsa_sparse_attn_decode": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _i32,
                                      ctypes.c_float, _c_p, _i64, _c_p, _c_p, _i64, _c_p, _sz, _c_p]),
    "qsa_index_select_decode_workspace_bytes": (_sz, [_i32, _i32]),
    "qsa_index_select_decode": (_i32, [_c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _i32, _c_p, _i64, _i64, _c_p,
                                       _i64, _c_p, _sz, _c_p]),
    "qsa_decode_step_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "qsa_decode_step": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _c_p, _i64, _c_p, _i64,
                               _c_p, _i64, _c_p, _i32, _i32, _i32, ctypes.c_float, _rope_p, _c_p, _i64,
                               _i64, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _i64, _c_p, _sz, _c_p]),
    "qsa_set_scan_timing_events": (_i32, [_c_p, _c_p]),
    "qsa_set_decode_fallback_counter": (_i32, [_c_p]),
    "qsa_decode_step_noalloc": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _c_p, _i64, _c_p,
                                       _i64, _c_p, _i64, _c_p, _i32, _i32, _i32, ctypes.c_float, _rope_p, _c_p,
                                       _i64, _i64, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _i64, _c_p]),
    "qsa_paged_append": (_i32, [_paged_p, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _rope_p, _c_p]),
    "qsa_index_select_prefill_paged": (_i32, [_c_p, _i64, _paged_p, _c_p, _i32, _i32, _i32, _c_p, _i64, _i64,
                                              _c_p, _i64, _c_p, _sz, _c_p]),
    "qsa_sparse_attn_prefill_paged": (_i32, [_c_p, _i64, _paged_p, _c_p, _i64, _c_p, _i32, _i32, _i32,
                                             ctypes.c_float, _c_p, _i64, _c_p, _i64, _c_p, _i64, _c_p]),
    "qsa_gdn_prefill_workspace_bytes": (_sz, [_i32, _i32]),
    "qsa_gdn_prefill": (_i32, [_c_p, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _i64, _c_p, _i32, _i32, _c_p, _i64,
                               _c_p, _sz, _c_p]),
    "qsa_gdn_decode": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p]),
    "qsa_decode_step_paged": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i64, _c_p, _paged_p, _c_p, _i32, _i32,
                                     _i32, ctypes.c_float, _rope_p, _c_p, _i64, _i64, _c_p, _i64, _c_p, _i64,
                                     _c_p, _c_p, _i64, _c_p, _sz, _c_p]),
}

EXPORTED = tuple(_SIGNATURES)


class QSAError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("block", "hq", "hkv", "d", "rot_dim", "hi", "di")]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so (built in-tree by block_sparse_long_12_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise QSAError(f"{LIB_PATH} is not built: run `python -m block_sparse_long_12_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.qsa_abi_version() != 4:
            raise QSAError("libqsa ABI version mismatch")
        _LIB = L
    return _LIB


def dims() -> dict:
    d = _Dims()
    _check(lib().qsa_get_dims(ctypes.byref(d)), "qsa_get_dims")
    return {n: getattr(d, n) for n, _ in _Dims._fields_}


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise QSAError(f"{what}: {L.qsa_status_string(status).decode()} "
                       f"({L.qsa_last_error().decode()})")


def _stream(stream) -> _c_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return _c_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None) -> _c_p:
    return _c_p(0 if t is None else t.data_ptr())


def _positions(pos, batch: int):
    vals = [int(x) for x in (pos.tolist() if hasattr(pos, "tolist") else pos)]
    if len(vals) != batch:
        raise QSAError(f"expected {batch} positions, got {len(vals)}")
    return (ctypes.c_int32 * batch)(*vals)


def _gate_args(gate, out: torch.Tensor):
    """(pointer, sequence stride) of an optional output gate laid out as out."""
    if gate is None:
        return _c_p(0), 0
    _need(gate, "gate", torch.bfloat16, (HQ, D))
    if tuple(gate.shape) != tuple(out.shape):
        raise QSAError("gate must have the shape of out")
    return _ptr(gate), gate.stride(0)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, inner: tuple[int, ...]) -> None:
    """t must be a device tensor of `dtype` whose dims after the first are
    packed: shape[1:] contiguous (the C ABI takes one stride per sequence)."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise QSAError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise QSAError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape[-len(inner):]) != inner and inner:
        raise QSAError(f"{name} trailing shape {tuple(t.shape)} does not end with {inner}")
    expect = 1
    for size, stride in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and stride != expect:
            raise QSAError(f"{name} must be packed after its first dimension")
        expect *= size


# ------------------------------------------------------------------ steps

def rope_apply(x: torch.Tensor, pos0, out: torch.Tensor | None = None,
               rope: Rope | None = None, stream=None) -> torch.Tensor:
    """Rotate dims 0..63 of x [B, T, H, 256] (bf16) at positions pos0[b] + t.
    out=None rotates in place; otherwise out [B, T, H, 256] receives the result.
    rope: rotary parameters (None: theta 1e7, no YaRN; YARN: the model card's
    static YaRN)."""
    _need(x, "x", torch.bfloat16, (D,))
    B, T, H = x.shape[0], x.shape[1], x.shape[2]
    y = x if out is None else out
    if out is not None:
        _need(out, "out", torch.bfloat16, (D,))
        if tuple(out.shape) != tuple(x.shape):
            raise QSAError("out must have the shape of x")
    _check(lib().qsa_rope_apply(_ptr(x), x.stride(0), x.stride(1), _ptr(y), y.stride(0), y.stride(1),
                                B, T, H, _positions(pos0, B), _rope_arg(rope), _stream(stream)),
           "qsa_rope_apply")
    return y


def compress_block_keys(k_idx: torch.Tensor, block_begin: int, block_end: int,
                        kbar: torch.Tensor, stream=None) -> torch.Tensor:
    """kbar[b, j] = bf16 mean of k_idx[b, 4j .. 4j+3] for j in [block_begin, block_end)."""
    _need(k_idx, "k_idx", torch.bfloat16, (DI,))
    _need(kbar, "kbar", torch.bfloat16, (DI,))
    B = k_idx.shape[0]
    if kbar.shape[0] != B or k_idx.shape[1] < BLOCK * block_end or kbar.shape[1] < block_end:
        raise QSAError("k_idx / kbar too short for block_end")
    _check(lib().qsa_compress_block_keys(_ptr(k_idx), k_idx.stride(0), B, block_begin, block_end,
                                         _ptr(kbar), kbar.stride(0), _stream(stream)),
           "qsa_compress_block_keys")
    return kbar


def index_scores(q_idx: torch.Tensor, kbar: torch.Tensor, q_pos0, scores: torch.Tensor,
                 stream=None) -> torch.Tensor:
    """scores[b, t, j] = sum_h q_idx[b, t, h] . kbar[b, j] for j < (q_pos0[b] + t) // 4."""
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(kbar, "kbar", torch.bfloat16, (DI,))
    _need(scores, "scores", torch.float32, ())
    B, T = q_idx.shape[0], q_idx.shape[1]
    pos = _positions(q_pos0, B)
    need = max((int(pos[b]) + T - 1) // BLOCK for b in range(B)) if T else 0
    if scores.shape[0] != B or scores.shape[1] < T or kbar.shape[0] != B or kbar.shape[1] < need:
        raise QSAError("scores / kbar shapes do not cover the queries")
    _check(lib().qsa_index_scores(_ptr(q_idx), q_idx.stride(0), _ptr(kbar), kbar.stride(0), pos, B, T,
                                  _ptr(scores), scores.stride(1), scores.stride(0), _stream(stream)),
           "qsa_index_scores")
    return scores


def select_topk(scores: torch.Tensor, q_pos0, budget: int, sel: torch.Tensor,
                stream=None) -> torch.Tensor:
    """sel[b, t] = ascending top-(budget-1) blocks by score plus the own block, -1 padded."""
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    B, T = sel.shape[0], sel.shape[1]
    if scores.shape[0] != B or scores.shape[1] < T:
        raise QSAError("scores does not cover sel's rows")
    L = lib()
    ws_bytes = L.qsa_select_workspace_bytes(B, T, budget)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=sel.device) if ws_bytes else None
    _check(L.qsa_select_topk(_ptr(scores), scores.stride(1), scores.stride(0), _positions(q_pos0, B), B, T,
                             budget, _ptr(sel), sel.stride(0), _ptr(ws), ws_bytes, _stream(stream)),
           "qsa_select_topk")
    return sel


def sparse_attn_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        sel: torch.Tensor, q_pos0, out: torch.Tensor, lse: torch.Tensor | None = None,
                        scale: float = 1.0 / math.sqrt(D), stream=None, gate=None) -> torch.Tensor:
    """out[b, t] = attention of q[b, t] (24 heads) over the tokens of sel[b, t];
    with gate (bf16, out's shape) each value is scaled by sigmoid(gate)."""
    _need(q, "q", torch.bfloat16, (HQ, D))
    _need(k_cache, "k_cache", torch.bfloat16, (HKV, D))
    _need(v_cache, "v_cache", torch.bfloat16, (HKV, D))
    _need(out, "out", torch.bfloat16, (HQ, D))
    B, T = q.shape[0], q.shape[1]
    budget = sel.shape[-1]
    _need(sel, "sel", torch.int32, (budget,))
    if lse is not None:
        _need(lse, "lse", torch.float32, (HQ,))
        if tuple(lse.shape) != (B, T, HQ):
            raise QSAError("lse must be [B, T, 24]")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise QSAError("k_cache and v_cache must share shape and strides")
    pos = _positions(q_pos0, B)
    if any(int(pos[b]) + T > k_cache.shape[1] for b in range(B)):
        raise QSAError("KV caches shorter than the query positions")
    g_ptr, g_stride = _gate_args(gate, out)
    _check(lib().qsa_sparse_attn_prefill(_ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), k_cache.stride(0),
                                         _ptr(sel), sel.stride(0), pos, B, T, budget, float(scale),
                                         _ptr(out), out.stride(0), _ptr(lse),
                                         0 if lse is None else lse.stride(0), g_ptr, g_stride, _stream(stream)),
           "qsa_sparse_attn_prefill")
    return out


def decode_workspace(batch: int, budget: int, device="cuda", tq: int = 1) -> torch.Tensor:
    """Workspace of sparse_attn_decode for batch sequences of tq decode tokens."""
    n = lib().qsa_decode_workspace_bytes(batch, tq, budget)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _decode_rows(q: torch.Tensor, inner: int) -> int:
    """tq of a decode tensor: [B, <inner dims>] is one token, [B, tq, <inner>] tq."""
    return 1 if q.dim() == 1 + inner else q.shape[1]


def sparse_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       sel: torch.Tensor, q_pos, out: torch.Tensor, lse: torch.Tensor | None,
                       workspace: torch.Tensor, scale: float = 1.0 / math.sqrt(D),
                       stream=None, gate=None) -> torch.Tensor:
    """Decode form: q [B, 24, 256] (or [B, tq, 24, 256]: tq consecutive tokens
    per sequence, token t at q_pos[b] + t), sel [B, budget] (or [B, tq, budget]),
    out like q, lse [B, 24] (or [B, tq, 24]), optional output gate like out."""
    _need(q, "q", torch.bfloat16, (HQ, D))
    _need(out, "out", torch.bfloat16, (HQ, D))
    _need(k_cache, "k_cache", torch.bfloat16, (HKV, D))
    _need(v_cache, "v_cache", torch.bfloat16, (HKV, D))
    B, tq, budget = q.shape[0], _decode_rows(q, 2), sel.shape[-1]
    _need(sel, "sel", torch.int32, (budget,))
    if tuple(out.shape) != tuple(q.shape) or sel.shape[0] != B or sel.numel() != B * tq * budget:
        raise QSAError("out must have the shape of q and sel hold [B, tq, budget]")
    if lse is not None and (not lse.is_contiguous() or lse.numel() != B * tq * HQ):
        raise QSAError("lse must be contiguous [B, tq, 24]")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise QSAError("k_cache and v_cache must share shape and strides")
    pos = _positions(q_pos, B)
    if any(int(pos[b]) + tq > k_cache.shape[1] for b in range(B)):
        raise QSAError("KV caches shorter than the query positions")
    g_ptr, g_stride = _gate_args(gate, out)
    _check(lib().qsa_sparse_attn_decode(_ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), k_cache.stride(0),
                                        _ptr(sel), sel.stride(0), pos, B, tq, budget, float(scale), _ptr(out),
                                        out.stride(0), _ptr(lse), g_ptr, g_stride, _ptr(workspace),
                                        workspace.numel(), _stream(stream)),
           "qsa_sparse_attn_decode")
    return out


# ------------------------------------------------------------------ chained steps

def index_select_prefill_workspace(batch: int, tq: int, device="cuda") -> torch.Tensor:
    """Workspace of the fused prefill index-select (any contents; reusable across calls)."""
    n = lib().qsa_index_select_prefill_workspace_bytes(batch, tq)
    return torch.empty(n, dtype=torch.uint8, device=device)


def index_select_prefill(q_idx: torch.Tensor, kbar: torch.Tensor, q_pos0, budget: int, scores: torch.Tensor,
                         sel: torch.Tensor, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Steps 2 + 3 for a prefill chunk (same result as index_scores + select_topk):
    q_idx [B, T, 4, 128], scores [B, >= T, ld] scratch, sel [B, T, budget]."""
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(kbar, "kbar", torch.bfloat16, (DI,))
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    B, T = q_idx.shape[0], q_idx.shape[1]
    pos = _positions(q_pos0, B)
    need = max((int(pos[b]) + T - 1) // BLOCK for b in range(B)) if T else 0
    if scores.shape[0] != B or scores.shape[1] < T or kbar.shape[0] != B or kbar.shape[1] < need:
        raise QSAError("scores / kbar shapes do not cover the queries")
    if sel.shape[0] != B or sel.shape[1] != T:
        raise QSAError("sel must be [B, T, budget]")
    _check(lib().qsa_index_select_prefill(_ptr(q_idx), q_idx.stride(0), _ptr(kbar), kbar.stride(0), pos, B, T,
                                          budget, _ptr(scores), scores.stride(1), scores.stride(0), _ptr(sel),
                                          sel.stride(0), _ptr(workspace), workspace.numel(), _stream(stream)),
           "qsa_index_select_prefill")
    return sel


class PrefillBuffers:
    """Device buffers for one prefill layer call: scratch scores for one query
    chunk, the fused index-select workspace and the per-token selection."""

    def __init__(self, batch: int, tq: int, ctx: int, budget: int, chunk: int | None, device="cuda"):
        self.chunk = min(tq, chunk or tq)
        ld = max(4, ((ctx + tq - 1) // BLOCK + 3) // 4 * 4)
        self.scores = torch.empty((batch, self.chunk, ld), dtype=torch.float32, device=device)
        self.sel = torch.empty((batch, tq, budget), dtype=torch.int32, device=device)
        self.workspace = index_select_prefill_workspace(batch, self.chunk, device=device)


def prefill_layer(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, q_pos0: int, budget: int,
                  out, lse, bufs: PrefillBuffers, q_rot, stream=None, gate=None, rope: Rope | None = None,
                  side_stream=None):
    """One QSA layer over tq new tokens of every sequence, all at q_pos0.

    q_raw [B, tq, 24, 256] and k_new_raw [B, tq, 2, 256] are unrotated; the
    rotated K rows are written into k_cache[:, q_pos0 : q_pos0 + tq] (V rows
    are expected in v_cache already, k_idx rows in k_idx).  Steps: rotary
    (Q -> q_rot, K -> cache), compress the blocks the chunk completes, then per
    query chunk the fused index-select, then attention (with the optional
    output gate [B, tq, 24, 256]).  rope: rotary parameters (see rope_apply).
    side_stream: when given, the query chunks' index-selects run in order on it
    and each chunk's attention (on `stream`) waits only for its own selection,
    so the selection of chunk c + 1 runs beside the attention of chunk c; the
    kernels and their results are the same.
    """
    B, tq = q_raw.shape[0], q_raw.shape[1]
    pos = [q_pos0] * B
    rope_apply(q_raw, pos, out=q_rot, rope=rope, stream=stream)
    rope_apply(k_new_raw, pos, out=k_cache[:, q_pos0:q_pos0 + tq], rope=rope, stream=stream)
    b0, b1 = q_pos0 // BLOCK, (q_pos0 + tq) // BLOCK
    compress_block_keys(k_idx, b0, b1, kbar, stream=stream)
    chunks = [(c0, min(tq, c0 + bufs.chunk)) for c0 in range(0, tq, bufs.chunk)]

    def select(c0, c1, st):
        index_select_prefill(q_idx[:, c0:c1], kbar, [q_pos0 + c0] * B, budget, bufs.scores,
                             bufs.sel[:, c0:c1], bufs.workspace, stream=st)

    def attend(c0, c1):
        sparse_attn_prefill(q_rot[:, c0:c1], k_cache, v_cache, bufs.sel[:, c0:c1], [q_pos0 + c0] * B,
                            out[:, c0:c1], None if lse is None else lse[:, c0:c1], stream=stream,
                            gate=None if gate is None else gate[:, c0:c1])

    _chunk_schedule(chunks, select, attend, stream, side_stream)
    return out


def _chunk_schedule(chunks, select, attend, stream, side_stream):
    """Run select(c0, c1, stream) then attend(c0, c1) for every query chunk.

    One stream: select and attend alternate on `stream`.  With side_stream:
    the selections run in order on side_stream (which first waits for the
    work already queued on `stream`) and each chunk's attention on `stream`
    waits on an event of its own selection, so selection c + 1 runs beside
    attention c.  The selections share one scratch workspace, which the
    in-order side stream makes safe; `stream` finally waits for side_stream."""
    if side_stream is None:
        for c0, c1 in chunks:
            select(c0, c1, stream)
            attend(c0, c1)
        return
    main = torch.cuda.current_stream() if stream is None else stream
    ready = torch.cuda.Event()
    ready.record(main)
    side_stream.wait_event(ready)                    # rotary, appends and block keys done
    done = []
    for c0, c1 in chunks:
        select(c0, c1, side_stream)
        e = torch.cuda.Event()
        e.record(side_stream)
        done.append(e)
    for (c0, c1), e in zip(chunks, done):
        main.wait_event(e)
        attend(c0, c1)
    main.wait_stream(side_stream)


def index_select_workspace(batch: int, device="cuda", tq: int = 1) -> torch.Tensor:
    """Zero-filled workspace of the fused decode index-select (reusable across calls)."""
    n = lib().qsa_index_select_decode_workspace_bytes(batch, tq)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def index_select_decode(q_idx: torch.Tensor, kbar: torch.Tensor, q_pos, budget: int, scores: torch.Tensor,
                        sel: torch.Tensor, workspace: torch.Tensor, stream=None):
    """Fused steps 2 + 3 for decode rows: q_idx [B, 4, 128] or [B, tq, 4, 128]
    (token t at q_pos[b] + t), scores [B, ld] or [B, tq, ld], sel [B, budget] or
    [B, tq, budget]."""
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(kbar, "kbar", torch.bfloat16, (DI,))
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    B, tq = q_idx.shape[0], _decode_rows(q_idx, 2)
    pos = _positions(q_pos, B)
    need = max((int(pos[b]) + tq - 1) // BLOCK for b in range(B))
    if scores.shape[-1] < need or kbar.shape[1] < need or scores.shape[-1] % 4:
        raise QSAError("scores / kbar do not cover the candidate blocks")
    if scores.numel() < B * tq * scores.shape[-1] or sel.numel() != B * tq * budget:
        raise QSAError("scores / sel must hold [B, tq, ...]")
    _check(lib().qsa_index_select_decode(_ptr(q_idx), q_idx.stride(0), _ptr(kbar), kbar.stride(0), pos, B, tq,
                                         budget, _ptr(scores), scores.shape[-1], scores.stride(0), _ptr(sel),
                                         sel.stride(0), _ptr(workspace), workspace.numel(), _stream(stream)),
           "qsa_index_select_decode")
    return sel


def decode_step_workspace(batch: int, budget: int, device="cuda", tq: int = 1) -> torch.Tensor:
    """Zero-filled workspace of qsa_decode_step (reusable across calls)."""
    n = lib().qsa_decode_step_workspace_bytes(batch, tq, budget)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _decode_positions(pos, B: int) -> list[int]:
    return [int(pos)] * B if isinstance(pos, int) else [int(x) for x in pos]


def decode_step(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, pos, budget: int,
                out, lse, scores, sel, workspace, stream=None, scale: float = 1.0 / math.sqrt(D),
                v_new=None, k_idx_new=None, gate=None, rope: Rope | None = None):
    """One decode step through the single qsa_decode_step call, for tq new
    tokens per sequence (tq = q_raw.shape[1], 1 .. 4): token t of sequence b
    at position pos[b] + t (pos an int: the same for all sequences).

    q_raw [B, tq, 24, 256] and k_new_raw [B, tq, 2, 256] are unrotated; the
    rotated K rows go to k_cache[b, pos[b] + t]. v_new [B, tq, 2, 256] and
    k_idx_new [B, tq, 128] (optional) are appended to v_cache / k_idx; without
    them those rows are expected in place. kbar must hold the blocks before
    pos[b] // 4; the step writes the key of every block a new token completes
    (from k_idx). rope: rotary parameters of q and the new K rows (see
    rope_apply). scores [B, tq, ld], sel [B, tq, budget], out [B, 24, 256]
    (tq = 1) or [B, tq, 24, 256], lse [B, 24] or [B, tq, 24], gate (optional
    output gate) like out. workspace comes from decode_step_workspace(B,
    budget, tq=tq).
    """
    B = q_raw.shape[0]
    p_list = _decode_positions(pos, B)
    _decode_step_check(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse, scores,
                       sel, v_new, k_idx_new)
    args = _decode_step_args(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse,
                             scores, sel, scale, v_new, k_idx_new, gate, rope)
    _check(lib().qsa_decode_step(*args, _ptr(workspace), workspace.numel(), _stream(stream)), "qsa_decode_step")
    return out


def _decode_step_args(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse, scores,
                      sel, scale, v_new, k_idx_new, gate, rope):
    """The C arguments of qsa_decode_step up to (not including) the workspace."""
    B, tq = q_raw.shape[0], q_raw.shape[1]
    p = _positions(p_list, B)
    g_ptr, g_stride = _gate_args(gate, out)
    return (_ptr(q_raw), q_raw.stride(0), _ptr(k_new_raw), _ptr(v_new), k_new_raw.stride(0),
            _ptr(q_idx), q_idx.stride(0), _ptr(k_idx_new), _ptr(k_cache), _ptr(v_cache),
            k_cache.stride(0), _ptr(k_idx), 0 if k_idx is None else k_idx.stride(0),
            _ptr(kbar), kbar.stride(0), p, B, tq, budget, float(scale), _rope_arg(rope),
            _ptr(scores), scores.shape[-1], scores.stride(0), _ptr(sel), sel.stride(0),
            _ptr(out), out.stride(0), _ptr(lse), g_ptr, g_stride)


def set_scan_timing_events(begin=None, end=None) -> None:
    """Measurement hook (qsa_set_scan_timing_events): while set, every decode
    index-select on this thread records the torch events `begin` / `end` (timing
    enabled, already recorded once so that torch considers them created) right
    before and after its block-key scan launch; None, None turns it off."""
    def handle(e):
        if e is None:
            return None
        h = int(e.cuda_event)
        if h == 0:
            raise QSAError("record the event once before handing it to the library")
        return h
    lib().qsa_set_scan_timing_events(handle(begin), handle(end))


def set_decode_fallback_counter(counter=None) -> None:
    """Diagnostic hook (qsa_set_decode_fallback_counter): while set, every
    decode index-select on this thread adds 1 to the one-element device tensor
    `counter` (int32 or uint32 storage) for each row that takes the exact path
    over the stored scores; None turns it off."""
    if counter is not None:
        if not (counter.is_cuda and counter.numel() == 1 and counter.element_size() == 4):
            raise QSAError("counter must be a one-element 4-byte device tensor")
    lib().qsa_set_decode_fallback_counter(None if counter is None else counter.data_ptr())


def decode_step_noalloc(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, pos, budget: int,
                        out, lse, scores, sel, stream=None, scale: float = 1.0 / math.sqrt(D),
                        v_new=None, k_idx_new=None, gate=None, rope: Rope | None = None):
    """decode_step without a workspace (qsa_decode_step_noalloc): the library's
    static per-GPU scratch serves instead, so the call allocates nothing.  Calls
    that overlap on one GPU race; shapes beyond the scratch raise QSAError."""
    B = q_raw.shape[0]
    p_list = _decode_positions(pos, B)
    _decode_step_check(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse, scores,
                       sel, v_new, k_idx_new)
    args = _decode_step_args(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse,
                             scores, sel, scale, v_new, k_idx_new, gate, rope)
    _check(lib().qsa_decode_step_noalloc(*args, _stream(stream)), "qsa_decode_step_noalloc")
    return out


def _decode_step_check(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, p_list, budget, out, lse, scores,
                       sel, v_new, k_idx_new):
    """Tensor checks of decode_step and decode_step_noalloc."""
    B, tq = q_raw.shape[0], q_raw.shape[1]
    _need(q_raw, "q", torch.bfloat16, (HQ, D))
    _need(k_new_raw, "k_new", torch.bfloat16, (HKV, D))
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(k_cache, "k_cache", torch.bfloat16, (HKV, D))
    _need(v_cache, "v_cache", torch.bfloat16, (HKV, D))
    _need(kbar, "kbar", torch.bfloat16, (DI,))
    _need(out, "out", torch.bfloat16, (HQ, D))
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    if k_new_raw.shape[1] != tq or q_idx.numel() != B * tq * HI * DI or out.numel() != B * tq * HQ * D:
        raise QSAError("k_new, q_idx and out must hold tq rows per sequence")
    if sel.numel() != B * tq * budget or scores.numel() < B * tq * scores.shape[-1]:
        raise QSAError("sel / scores must hold [B, tq, ...]")
    if k_idx is not None:
        _need(k_idx, "k_idx", torch.bfloat16, (DI,))
    if v_new is not None:
        _need(v_new, "v_new", torch.bfloat16, (HKV, D))
        if v_new.stride(0) != k_new_raw.stride(0) or v_new.shape[1] != tq:
            raise QSAError("v_new must match k_new in shape and sequence stride")
    if k_idx_new is not None:
        if k_idx is None:
            raise QSAError("k_idx_new needs the k_idx cache")
        if (not isinstance(k_idx_new, torch.Tensor) or k_idx_new.device.type != "cuda"
                or k_idx_new.dtype != torch.bfloat16 or not k_idx_new.is_contiguous()
                or k_idx_new.numel() != B * tq * DI):
            raise QSAError("k_idx_new must be a contiguous bf16 device tensor [B, tq, 128]")
    top = max(p_list) + tq - 1
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape or k_cache.shape[1] <= top:
        raise QSAError("k_cache / v_cache must share shape and strides and hold every new position")
    if k_idx is not None and k_idx.shape[1] <= top:
        raise QSAError("k_idx must hold every new position")
    if lse is not None and (not lse.is_contiguous() or lse.numel() != B * tq * HQ):
        raise QSAError("lse must be contiguous [B, tq, 24]")
    if scores.shape[-1] < top // BLOCK or scores.shape[-1] % 4:
        raise QSAError("scores do not cover the candidate blocks")
    if kbar.shape[1] < max((x + tq) // BLOCK if k_idx is not None else (x + tq - 1) // BLOCK for x in p_list):
        raise QSAError("kbar does not cover the candidate (and completed) blocks")


def decode_step_primitives(q_raw, k_new_raw, q_idx, k_idx, k_cache, v_cache, kbar, pos, budget: int,
                           out, lse, scores, sel, workspace, q_rot, stream=None, v_new=None, k_idx_new=None,
                           gate=None, rope: Rope | None = None):
    """The same decode step as a chain of the primitive calls (rotary, row
    copies, block compression, scores, selection, attention); workspace from
    decode_workspace(B, budget, tq=tq)."""
    B, tq = q_raw.shape[0], q_raw.shape[1]
    p = _decode_positions(pos, B)
    rope_apply(q_raw, p, out=q_rot, rope=rope, stream=stream)
    for b in range(B):
        rope_apply(k_new_raw[b:b + 1], [p[b]], out=k_cache[b:b + 1, p[b]:p[b] + tq], rope=rope, stream=stream)
        if v_new is not None:
            v_cache[b, p[b]:p[b] + tq].copy_(v_new[b])
        if k_idx_new is not None:
            k_idx[b, p[b]:p[b] + tq].copy_(k_idx_new.reshape(B, tq, DI)[b])
    if k_idx is not None:
        for b in range(B):
            j0, j1 = p[b] // BLOCK, (p[b] + tq) // BLOCK            # blocks j with 4j + 3 in [p, p + tq)
            if j1 > j0:
                compress_block_keys(k_idx[b:b + 1], j0, j1, kbar[b:b + 1], stream=stream)
    index_scores(q_idx, kbar, p, scores, stream=stream)
    select_topk(scores, p, budget, sel, stream=stream)
    q_att = q_rot if tq > 1 else q_rot[:, 0]
    sel_att = sel if tq > 1 else sel[:, 0]
    sparse_attn_decode(q_att, k_cache, v_cache, sel_att, p, out, lse, workspace, stream=stream, gate=gate)
    return out


# ------------------------------------------------------------------ paged caches

class PagedCache:
    """Paged caches with a block table (device tensors): k, v [n_pages, P, 2, 256],
    k_idx [n_pages, P, 128], kbar [n_pages, P/4, 128] and table int32
    [batch, max_pages]: token n of sequence b sits in page table[b, n // P],
    row n % P.  Sequences may share the pages of a common prefix."""

    def __init__(self, n_pages: int, page_tokens: int, batch: int, max_pages: int, device="cuda",
                 with_k_idx: bool = True):
        P = int(page_tokens)
        if P < 64 or P & (P - 1):
            raise QSAError("page_tokens must be a power of two >= 64")
        bf = torch.bfloat16
        self.page_tokens, self.n_pages = P, int(n_pages)
        self.k = torch.zeros((n_pages, P, HKV, D), dtype=bf, device=device)
        self.v = torch.zeros_like(self.k)
        self.k_idx = torch.zeros((n_pages, P, DI), dtype=bf, device=device) if with_k_idx else None
        self.kbar = torch.zeros((n_pages, P // BLOCK, DI), dtype=bf, device=device)
        self.table = torch.zeros((batch, max_pages), dtype=torch.int32, device=device)

    def _rows(self, b: int, n_tok: int) -> torch.Tensor:
        n = torch.arange(n_tok, device=self.table.device)
        return self.table[b][n // self.page_tokens].long() * self.page_tokens + n % self.page_tokens

    def _blocks(self, b: int, n_blk: int) -> torch.Tensor:
        j = torch.arange(n_blk, device=self.table.device)
        per = self.page_tokens // BLOCK
        return self.table[b][(BLOCK * j) // self.page_tokens].long() * per + j % per

    def write_contiguous(self, b: int, upto: int, k=None, v=None, k_idx=None, kbar=None) -> None:
        """Copy tokens 0 .. upto - 1 of sequence b from contiguous caches
        (k, v [L, 2, 256], k_idx [L, 128]) and the keys of its complete blocks
        (kbar [L/4, 128]) into the pages its table row names."""
        r = self._rows(b, upto)
        if k is not None:
            self.k.view(-1, HKV, D)[r] = k[:upto]
        if v is not None:
            self.v.view(-1, HKV, D)[r] = v[:upto]
        if k_idx is not None:
            self.k_idx.view(-1, DI)[r] = k_idx[:upto]
        if kbar is not None and upto // BLOCK:
            self.kbar.view(-1, DI)[self._blocks(b, upto // BLOCK)] = kbar[:upto // BLOCK]

    def read_contiguous(self, b: int, n_tok: int):
        """Tokens 0 .. n_tok - 1 of sequence b (k, v, k_idx) and the keys of its
        complete blocks, gathered from the pages into new tensors."""
        r = self._rows(b, n_tok)
        k_idx = None if self.k_idx is None else self.k_idx.view(-1, DI)[r]
        return (self.k.view(-1, HKV, D)[r], self.v.view(-1, HKV, D)[r], k_idx,
                self.kbar.view(-1, DI)[self._blocks(b, n_tok // BLOCK)])

    def c_struct(self) -> _PagedCacheC:
        for name in ("k", "v", "kbar", "table"):
            t = getattr(self, name)
            if not t.is_contiguous():
                raise QSAError(f"paged cache {name} must be contiguous")
        return _PagedCacheC(self.k.data_ptr(), self.v.data_ptr(),
                            0 if self.k_idx is None else self.k_idx.data_ptr(), self.kbar.data_ptr(),
                            self.table.data_ptr(), self.table.stride(0), self.page_tokens, self.n_pages)


def paged_append(cache: PagedCache, pos0, k_new=None, v_new=None, k_idx_new=None, rope: Rope | None = None,
                 stream=None) -> None:
    """Write the new tokens pos0[b] .. pos0[b] + T - 1 into their pages: k_new
    [B, T, 2, 256] rotated (as rope_apply), v_new [B, T, 2, 256], k_idx_new
    [B, T, 128] (None: skipped), then the key of every block they complete."""
    ref = next((t for t in (k_new, v_new, k_idx_new) if t is not None), None)
    if ref is None:
        raise QSAError("paged_append needs at least one of k_new, v_new, k_idx_new")
    B, T = ref.shape[0], ref.shape[1]
    for t, name, inner in ((k_new, "k_new", (HKV, D)), (v_new, "v_new", (HKV, D)), (k_idx_new, "k_idx_new", (DI,))):
        if t is not None:
            _need(t, name, torch.bfloat16, inner)
            if t.shape[0] != B or t.shape[1] != T:
                raise QSAError(f"{name} must be [B, T, ...] like the other new rows")
    if k_new is not None and v_new is not None and k_new.stride(0) != v_new.stride(0):
        raise QSAError("k_new and v_new must share the sequence stride")
    kv = k_new if k_new is not None else v_new
    c = cache.c_struct()
    _check(lib().qsa_paged_append(ctypes.byref(c), _ptr(k_new), _ptr(v_new), 0 if kv is None else kv.stride(0),
                                  _ptr(k_idx_new), 0 if k_idx_new is None else k_idx_new.stride(0),
                                  _positions(pos0, B), B, T, _rope_arg(rope), _stream(stream)),
           "qsa_paged_append")


def index_select_prefill_paged(q_idx: torch.Tensor, cache: PagedCache, q_pos0, budget: int, scores: torch.Tensor,
                               sel: torch.Tensor, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """index_select_prefill with the block keys in the paged cache."""
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    B, T = q_idx.shape[0], q_idx.shape[1]
    if scores.shape[0] != B or scores.shape[1] < T or sel.shape[0] != B or sel.shape[1] != T:
        raise QSAError("scores / sel shapes do not cover the queries")
    c = cache.c_struct()
    _check(lib().qsa_index_select_prefill_paged(_ptr(q_idx), q_idx.stride(0), ctypes.byref(c), _positions(q_pos0, B),
                                                B, T, budget, _ptr(scores), scores.stride(1), scores.stride(0),
                                                _ptr(sel), sel.stride(0), _ptr(workspace), workspace.numel(),
                                                _stream(stream)),
           "qsa_index_select_prefill_paged")
    return sel


def sparse_attn_prefill_paged(q: torch.Tensor, cache: PagedCache, sel: torch.Tensor, q_pos0, out: torch.Tensor,
                              lse: torch.Tensor | None = None, scale: float = 1.0 / math.sqrt(D), stream=None,
                              gate=None) -> torch.Tensor:
    """sparse_attn_prefill with K / V gathered from the paged cache."""
    _need(q, "q", torch.bfloat16, (HQ, D))
    _need(out, "out", torch.bfloat16, (HQ, D))
    B, T = q.shape[0], q.shape[1]
    budget = sel.shape[-1]
    _need(sel, "sel", torch.int32, (budget,))
    if lse is not None:
        _need(lse, "lse", torch.float32, (HQ,))
        if tuple(lse.shape) != (B, T, HQ):
            raise QSAError("lse must be [B, T, 24]")
    g_ptr, g_stride = _gate_args(gate, out)
    c = cache.c_struct()
    _check(lib().qsa_sparse_attn_prefill_paged(_ptr(q), q.stride(0), ctypes.byref(c), _ptr(sel), sel.stride(0),
                                               _positions(q_pos0, B), B, T, budget, float(scale), _ptr(out),
                                               out.stride(0), _ptr(lse), 0 if lse is None else lse.stride(0),
                                               g_ptr, g_stride, _stream(stream)),
           "qsa_sparse_attn_prefill_paged")
    return out


def decode_step_paged(q_raw, k_new_raw, q_idx, cache: PagedCache, pos, budget: int, out, lse, scores, sel,
                      workspace, stream=None, scale: float = 1.0 / math.sqrt(D), v_new=None, k_idx_new=None,
                      gate=None, rope: Rope | None = None):
    """decode_step on the paged cache (same arguments, the caches replaced by
    `cache`); workspace from decode_step_workspace(B, budget, tq=tq)."""
    B, tq = q_raw.shape[0], q_raw.shape[1]
    p_list = _decode_positions(pos, B)
    _need(q_raw, "q", torch.bfloat16, (HQ, D))
    _need(k_new_raw, "k_new", torch.bfloat16, (HKV, D))
    _need(q_idx, "q_idx", torch.bfloat16, (HI, DI))
    _need(out, "out", torch.bfloat16, (HQ, D))
    _need(scores, "scores", torch.float32, ())
    _need(sel, "sel", torch.int32, (budget,))
    if k_new_raw.shape[1] != tq or q_idx.numel() != B * tq * HI * DI or out.numel() != B * tq * HQ * D:
        raise QSAError("k_new, q_idx and out must hold tq rows per sequence")
    if sel.numel() != B * tq * budget or scores.numel() < B * tq * scores.shape[-1]:
        raise QSAError("sel / scores must hold [B, tq, ...]")
    if v_new is not None:
        _need(v_new, "v_new", torch.bfloat16, (HKV, D))
        if v_new.stride(0) != k_new_raw.stride(0) or v_new.shape[1] != tq:
            raise QSAError("v_new must match k_new in shape and sequence stride")
    if k_idx_new is not None and (not isinstance(k_idx_new, torch.Tensor) or k_idx_new.device.type != "cuda"
                                  or k_idx_new.dtype != torch.bfloat16 or not k_idx_new.is_contiguous()
                                  or k_idx_new.numel() != B * tq * DI):
        raise QSAError("k_idx_new must be a contiguous bf16 device tensor [B, tq, 128]")
    if lse is not None and (not lse.is_contiguous() or lse.numel() != B * tq * HQ):
        raise QSAError("lse must be contiguous [B, tq, 24]")
    g_ptr, g_stride = _gate_args(gate, out)
    c = cache.c_struct()
    _check(lib().qsa_decode_step_paged(_ptr(q_raw), q_raw.stride(0), _ptr(k_new_raw), _ptr(v_new),
                                       k_new_raw.stride(0), _ptr(q_idx), q_idx.stride(0), _ptr(k_idx_new),
                                       ctypes.byref(c), _positions(p_list, B), B, tq, budget, float(scale),
                                       _rope_arg(rope), _ptr(scores), scores.shape[-1], scores.stride(0), _ptr(sel),
                                       sel.stride(0), _ptr(out), out.stride(0), _ptr(lse), g_ptr, g_stride,
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "qsa_decode_step_paged")
    return out


def prefill_layer_paged(q_raw, k_new_raw, v_new, q_idx, k_idx_new, cache: PagedCache, q_pos0: int, budget: int,
                        out, lse, bufs: PrefillBuffers, q_rot, stream=None, gate=None, rope: Rope | None = None,
                        side_stream=None):
    """prefill_layer on the paged cache: the new K (rotated), V and indexer-key
    rows are written into their pages with the keys of the blocks they
    complete (paged_append), then per query chunk the fused index-select and
    attention read through the block table.  side_stream: the two-stream
    order of prefill_layer (same kernels, same results)."""
    B, tq = q_raw.shape[0], q_raw.shape[1]
    pos = [q_pos0] * B
    rope_apply(q_raw, pos, out=q_rot, rope=rope, stream=stream)
    paged_append(cache, pos, k_new=k_new_raw, v_new=v_new, k_idx_new=k_idx_new, rope=rope, stream=stream)
    chunks = [(c0, min(tq, c0 + bufs.chunk)) for c0 in range(0, tq, bufs.chunk)]

    def select(c0, c1, st):
        index_select_prefill_paged(q_idx[:, c0:c1], cache, [q_pos0 + c0] * B, budget, bufs.scores,
                                   bufs.sel[:, c0:c1], bufs.workspace, stream=st)

    def attend(c0, c1):
        sparse_attn_prefill_paged(q_rot[:, c0:c1], cache, bufs.sel[:, c0:c1], [q_pos0 + c0] * B, out[:, c0:c1],
                                  None if lse is None else lse[:, c0:c1], stream=stream,
                                  gate=None if gate is None else gate[:, c0:c1])

    _chunk_schedule(chunks, select, attend, stream, side_stream)
    return out


# ------------------------------------------------------------------ Gated DeltaNet

GDN_HK, GDN_HV, GDN_D = 16, 48, 128


def gdn_prefill_workspace(batch: int, n_tokens: int, device="cuda") -> torch.Tensor:
    """Workspace of gdn_prefill (no initialisation needed)."""
    n = lib().qsa_gdn_prefill_workspace_bytes(batch, n_tokens)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _gdn_check(q, k, v, g, beta, state, out, tok_dims):
    for t, name, dt, inner in ((q, "q", torch.bfloat16, (GDN_HK, GDN_D)), (k, "k", torch.bfloat16, (GDN_HK, GDN_D)),
                               (v, "v", torch.bfloat16, (GDN_HV, GDN_D)), (out, "out", torch.bfloat16, (GDN_HV, GDN_D)),
                               (g, "g", torch.float32, (GDN_HV,)), (beta, "beta", torch.float32, (GDN_HV,))):
        _need(t, name, dt, inner)
        if t.shape[:tok_dims] != q.shape[:tok_dims]:
            raise QSAError(f"{name} must match q in its leading dims")
    if q.stride() != k.stride() or g.stride() != beta.stride():
        raise QSAError("q / k and g / beta must share strides")
    _need(state, "state", torch.float32, (GDN_HV, GDN_D, GDN_D))
    if not state.is_contiguous() or state.shape[0] != q.shape[0]:
        raise QSAError("state must be contiguous [B, 48, 128, 128]")


def gdn_prefill(q, k, v, g, beta, state, out, workspace, stream=None):
    """Gated DeltaNet over T tokens per sequence: q, k [B, T, 16, 128], v and out
    [B, T, 48, 128] (bf16), g and beta [B, T, 48] (float32), state [B, 48, 128,
    128] (float32, updated in place to the state after the T tokens)."""
    _gdn_check(q, k, v, g, beta, state, out, 2)
    B, T = q.shape[0], q.shape[1]
    _check(lib().qsa_gdn_prefill(_ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0), _ptr(g), _ptr(beta),
                                 g.stride(0), _ptr(state), B, T, _ptr(out), out.stride(0), _ptr(workspace),
                                 workspace.numel(), _stream(stream)),
           "qsa_gdn_prefill")
    return out


def gdn_decode(q, k, v, g, beta, state, out, stream=None):
    """One Gated DeltaNet token per sequence: q, k [B, 16, 128], v and out
    [B, 48, 128], g and beta [B, 48]; state updated in place."""
    _gdn_check(q, k, v, g, beta, state, out, 1)
    for t in (q, k, v, g, beta, out):
        if not t.is_contiguous():
            raise QSAError("gdn_decode takes contiguous tensors")
    _check(lib().qsa_gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), q.shape[0], _ptr(out),
                                _stream(stream)),
           "qsa_gdn_decode")
    return out
