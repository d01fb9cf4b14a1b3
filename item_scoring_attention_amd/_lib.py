"""ctypes binding of ``libmis.so`` (declared in ``include/mis.h``).

Argument marshalling only: torch tensors become device pointers and the
current HIP stream, numpy/int sequences become host int32 arrays, and status
codes become exceptions (``ValueError`` for argument, segment and label
errors, ``RuntimeError`` otherwise). Every step of the computation runs in
the HIP library; there is no fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmis.so")

MIS_OK = 0
MIS_ERR_ARG = -1
MIS_ERR_SEGMENTS = -2
MIS_ERR_LABEL = -3
MIS_ERR_WORKSPACE = -4
MIS_ERR_UNSUPPORTED = -5
MIS_ERR_HIP = -6
MIS_MAX_LABELS = 256
MIS_SCORE_SCRATCH_BYTES = 16 << 20

MIS_F32 = 0
MIS_BF16 = 1

_ERR_NAMES = {
    MIS_ERR_ARG: "MIS_ERR_ARG",
    MIS_ERR_SEGMENTS: "MIS_ERR_SEGMENTS",
    MIS_ERR_LABEL: "MIS_ERR_LABEL",
    MIS_ERR_WORKSPACE: "MIS_ERR_WORKSPACE",
    MIS_ERR_UNSUPPORTED: "MIS_ERR_UNSUPPORTED",
    MIS_ERR_HIP: "MIS_ERR_HIP",
}

_i32p = ctypes.c_void_p  # host int32 arrays are passed by address
_i8p = ctypes.POINTER(ctypes.c_int8)


class MisSegments(ctypes.Structure):
    """Mirror of ``mis_segments`` (host struct holding device pointers)."""

    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("total_items", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("num_tiles", ctypes.c_int32),
        ("num_work", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("num_visits", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("prefix_lens", ctypes.c_void_p),
        ("cu_items", ctypes.c_void_p),
        ("cu_tiles", ctypes.c_void_p),
        ("item_begin", ctypes.c_void_p),
        ("readout_pos", ctypes.c_void_p),
        ("item_id", ctypes.c_void_p),
        ("pos_id", ctypes.c_void_p),
        ("tile_class", ctypes.c_void_p),
        ("work", ctypes.c_void_p),
    ]


# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "mis_segments_bytes": (ctypes.c_int, [ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "mis_build_segments": (ctypes.c_int, [ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.POINTER(MisSegments), ctypes.c_void_p]),
    "mis_attention_tile_shape": (ctypes.c_int, [ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, _i32p, _i32p]),
    "mis_attention_prefill": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]),
    "mis_attention_append": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]),
    "mis_apply_rope": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_float, ctypes.c_void_p]),
    "mis_rope_table_bytes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "mis_rope_table": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]),
    "mis_attention_prefill_rope": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                  ctypes.c_int32, ctypes.c_void_p]),
    "mis_attention_append_rope": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_void_p]),
    "mis_score_workspace_bytes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "mis_score_labels": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int, _i32p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mis_score_labels_noalloc": (ctypes.c_int, [ctypes.POINTER(MisSegments), ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_void_p, ctypes.c_int32, ctypes.c_int, _i32p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p]),
    "mis_score_labels_at": (ctypes.c_int, [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int,
                                           _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mis_set_kernel_choice": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p]),
    "mis_attention_kernel_name": (ctypes.c_char_p, [ctypes.POINTER(MisSegments), ctypes.c_int, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32]),
    "mis_score_kernel_name": (ctypes.c_char_p, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int]),
    "mis_last_error": (ctypes.c_char_p, []),
    "mis_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m item_scoring_attention_amd.build or __graft_entry__.build())"
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MisError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class MisValueError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc == MIS_OK:
        return
    msg = load().mis_last_error().decode()
    if rc in (MIS_ERR_ARG, MIS_ERR_SEGMENTS, MIS_ERR_LABEL):
        raise MisValueError(rc, msg)
    raise MisError(rc, msg)


def _host_i32(x) -> np.ndarray:
    if isinstance(x, np.ndarray) and x.dtype == np.int32 and x.flags.c_contiguous:
        return x
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    if a.size and (a.min() < -(2**31) or a.max() > 2**31 - 1):
        raise ValueError("metadata value outside int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _ptr_i32(a: Optional[np.ndarray]):
    """Address of a host int32 array (or None) for a ``const int32_t *`` parameter."""
    if a is None or a.size == 0:
        return None
    return a.ctypes.data


def _torch():
    import torch

    return torch


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MIS_BF16
    if t.dtype == torch.float32:
        return MIS_F32
    raise ValueError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def version() -> str:
    return load().mis_version().decode()


def set_kernel_choice(attention: Optional[str] = None, score: Optional[str] = None) -> None:
    """Force the attention / scoring kernel variant of this thread's later
    calls (``None`` or ``"auto"``: picked by shape); see ``include/mis.h``."""
    enc = lambda x: None if x is None else x.encode()
    _check(load().mis_set_kernel_choice(enc(attention), enc(score)))


def _code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    torch = _torch()
    return MIS_BF16 if dtype == torch.bfloat16 else MIS_F32


def attention_kernel_name(seg: "Segments", dtype, hq: int, hkv: int, head_dim: int) -> str:
    """The kernel ``mis_attention_prefill`` launches on this thread for these arguments."""
    name = load().mis_attention_kernel_name(ctypes.byref(seg.struct), _code(dtype), int(hq), int(hkv),
                                            int(head_dim)).decode()
    if not name:
        raise MisValueError(MIS_ERR_ARG, last_error())
    return name


def score_kernel_name(num_items: int, hidden_size: int, dtype) -> str:
    """The LM-head kernel ``mis_score_labels`` launches on this thread for this shape."""
    name = load().mis_score_kernel_name(int(num_items), int(hidden_size), _code(dtype)).decode()
    if not name:
        raise MisValueError(MIS_ERR_ARG, last_error())
    return name


def last_error() -> str:
    return load().mis_last_error().decode()


# ---------------------------------------------------------------- segments


class Segments:
    """Built segment descriptors: the C struct plus the device buffer it points into."""

    def __init__(self, struct: MisSegments, buf):
        self.struct = struct
        self.buf = buf  # keeps the device memory alive

    def __getattr__(self, name):
        if name in ("struct", "buf"):
            raise AttributeError(name)
        return getattr(self.struct, name)

    def array(self, name: str):
        """Device tensor view of one descriptor array (int32, or int8 for tile_class)."""
        torch = _torch()
        s = self.struct
        n = {
            "cu_seqlens": s.num_requests + 1,
            "prefix_lens": s.num_requests,
            "cu_items": s.num_requests + 1,
            "cu_tiles": s.num_requests + 1,
            "item_begin": s.total_items,
            "readout_pos": s.total_items,
            "item_id": s.total_tokens,
            "pos_id": s.total_tokens,
            "tile_class": s.num_tiles,
            "work": 4 * s.num_work,
        }[name]
        off = getattr(s, name) - self.buf.data_ptr()
        if name == "tile_class":
            return self.buf[off : off + n].view(torch.int8)
        return self.buf[off : off + 4 * n].view(torch.int32)


def mis_segments_bytes(cu_seqlens, total_items: int, block_m: int, block_n: int) -> int:
    cu = _host_i32(cu_seqlens)
    out = ctypes.c_size_t(0)
    _check(load().mis_segments_bytes(len(cu) - 1, _ptr_i32(cu), int(total_items), int(block_m),
                                     int(block_n), ctypes.byref(out)))
    return out.value


def mis_build_segments(cu_seqlens, prefix_lens, cu_items, item_starts, block_m: int, block_n: int,
                       dev_buf=None, stream=None, device=None) -> Segments:
    """Build segment descriptors; allocates ``dev_buf`` with torch when not given."""
    torch = _torch()
    cu = _host_i32(cu_seqlens)
    pl = _host_i32(prefix_lens)
    ci = _host_i32(cu_items)
    st = _host_i32(item_starts)
    B = len(cu) - 1
    if dev_buf is None:
        nbytes = mis_segments_bytes(cu, int(ci[-1]) if len(ci) else 0, block_m, block_n)
        dev_buf = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
    out = MisSegments()
    _check(load().mis_build_segments(B, _ptr_i32(cu), _ptr_i32(pl), _ptr_i32(ci), _ptr_i32(st),
                                     int(block_m), int(block_n),
                                     ctypes.c_void_p(dev_buf.data_ptr()),
                                     dev_buf.numel() * dev_buf.element_size(), ctypes.byref(out),
                                     _stream(stream)))
    return Segments(out, dev_buf)


# ---------------------------------------------------------------- attention


def mis_attention_tile_shape(dtype, hq: int, hkv: int, head_dim: int):
    torch = _torch()
    code = dtype if isinstance(dtype, int) else (MIS_BF16 if dtype == torch.bfloat16 else MIS_F32)
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().mis_attention_tile_shape(code, int(hq), int(hkv), int(head_dim),
                                           ctypes.addressof(bm), ctypes.addressof(bn)))
    return bm.value, bn.value


def mis_attention_prefill(seg: Segments, q, k, v, o=None, softmax_scale: float = 0.0, stream=None):
    """MIS attention. q ``[T,Hq,D]``, k/v ``[T,Hkv,D]``; returns o ``[T,Hq,D]``."""
    return _attention("mis_attention_prefill", seg, q, k, v, o, softmax_scale, stream)


def mis_attention_append(seg: Segments, q, k, v, o, softmax_scale: float = 0.0, stream=None):
    """Item rows only against a cached prefix (prefix rows of ``o`` are not recomputed)."""
    return _attention("mis_attention_append", seg, q, k, v, o, softmax_scale, stream)


def mis_attention_prefill_rope(seg: Segments, q, k, v, rope_table, o=None, softmax_scale: float = 0.0,
                               stream=None):
    """``mis_attention_prefill`` with Q rotated inside the kernel: q is Q before
    rotation (left unchanged), k already rotated, rope_table from
    ``mis_rope_table`` with at least ``seg.max_seqlen`` positions."""
    return _attention("mis_attention_prefill_rope", seg, q, k, v, o, softmax_scale, stream, rope_table)


def mis_attention_append_rope(seg: Segments, q, k, v, o, rope_table, softmax_scale: float = 0.0, stream=None):
    """``mis_attention_append`` with Q rotated inside the kernel (see
    ``mis_attention_prefill_rope``)."""
    return _attention("mis_attention_append_rope", seg, q, k, v, o, softmax_scale, stream, rope_table)


def _attention(fn: str, seg: Segments, q, k, v, o, softmax_scale: float, stream, rope_table=None):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, heads, D]")
    if k.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("k and v must match in shape, and q/k/v in dtype")
    if q.shape[0] != seg.total_tokens or k.shape[0] != seg.total_tokens:
        raise ValueError("token count of q/k/v differs from the segments")
    if q.shape[2] != k.shape[2]:
        raise ValueError("head_dim of q and k differ")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    args = [ctypes.byref(seg.struct), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dtype_code(q),
            q.shape[1], k.shape[1], q.shape[2], float(softmax_scale)]
    if rope_table is not None:
        if rope_table.dtype != torch.float32 or rope_table.dim() != 2 or rope_table.shape[1] != q.shape[2]:
            raise ValueError("rope_table must be float32 [positions, head_dim] from mis_rope_table")
        args += [_dev(rope_table, "rope_table"), rope_table.shape[0]]
    _check(getattr(load(), fn)(*args, _stream(stream)))
    return o


def mis_apply_rope(seg: Segments, q, k, theta: float, stream=None):
    """Rotary embedding of q ``[T,Hq,D]`` and k ``[T,Hkv,D]`` in place at the
    segment position ids; returns (q, k). ``q=None`` rotates k alone (for the
    ``*_rope`` attention calls, which rotate Q themselves)."""
    if (q is not None and q.dim() != 3) or k.dim() != 3:
        raise ValueError("q and k must be [T, heads, D]")
    if q is not None and q.dtype != k.dtype:
        raise ValueError("q and k must have the same dtype")
    if k.shape[0] != seg.total_tokens or (q is not None and q.shape[0] != seg.total_tokens):
        raise ValueError("token count of q/k differs from the segments")
    if q is not None and q.shape[2] != k.shape[2]:
        raise ValueError("head_dim of q and k differ")
    hq = q.shape[1] if q is not None else k.shape[1]
    _check(load().mis_apply_rope(ctypes.byref(seg.struct), _dev(q, "q") if q is not None else None, _dev(k, "k"),
                                 _dtype_code(k), hq, k.shape[1], k.shape[2], float(theta), _stream(stream)))
    return q, k


def mis_rope_table_bytes(num_positions: int, head_dim: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mis_rope_table_bytes(int(num_positions), int(head_dim), ctypes.byref(out)))
    return out.value


def mis_rope_table(num_positions: int, head_dim: int, theta: float, table=None, device=None, stream=None):
    """Rotary table float32 ``[num_positions, head_dim]``: (cos, sin) of pair i
    of position p at ``[p, 2i]``, ``[p, 2i+1]``; see ``include/mis.h``."""
    torch = _torch()
    nbytes = mis_rope_table_bytes(num_positions, head_dim)
    if table is None:
        table = torch.empty((int(num_positions), int(head_dim)), dtype=torch.float32,
                            device=device if device is not None else "cuda")
    elif table.dtype != torch.float32 or table.numel() * 4 < nbytes:
        raise ValueError("table must be float32 with at least num_positions x head_dim elements")
    _check(load().mis_rope_table(int(num_positions), int(head_dim), float(theta), _dev(table, "table"),
                                 table.numel() * 4, _stream(stream)))
    return table


# ---------------------------------------------------------------- scoring


def mis_score_workspace_bytes(num_items: int, vocab: int, num_labels: int, hidden: int,
                              dtype) -> int:
    torch = _torch()
    code = dtype if isinstance(dtype, int) else (MIS_BF16 if dtype == torch.bfloat16 else MIS_F32)
    out = ctypes.c_size_t(0)
    _check(load().mis_score_workspace_bytes(int(num_items), int(vocab), int(num_labels), int(hidden),
                                            code, ctypes.byref(out)))
    return out.value


def mis_score_labels(seg: Segments, hidden, lm_head, label_ids: Sequence[int],
                     apply_softmax: bool = False, scores=None, ws=None, stream=None):
    """Label scores ``[N, K]`` (float32) of every item; see ``include/mis.h``."""
    torch = _torch()
    if hidden.dim() != 2 or lm_head.dim() != 2 or hidden.shape[1] != lm_head.shape[1]:
        raise ValueError("hidden must be [T, H] and lm_head [V, H]")
    if hidden.shape[0] != seg.total_tokens:
        raise ValueError("hidden rows differ from the segments' token count")
    if hidden.dtype != lm_head.dtype:
        raise ValueError("hidden and lm_head dtypes differ")
    lab = _host_i32(label_ids)
    N, K = seg.total_items, len(lab)
    H, V = hidden.shape[1], lm_head.shape[0]
    if scores is None:
        scores = torch.empty((N, K), dtype=torch.float32, device=hidden.device)
    elif scores.dtype != torch.float32 or tuple(scores.shape) != (N, K):
        raise ValueError("scores must be float32 [N, K]")
    if ws is None:
        nbytes = mis_score_workspace_bytes(N, V, max(K, 1), H, hidden.dtype) if K >= 1 else 256
        ws = torch.empty(nbytes, dtype=torch.uint8, device=hidden.device)
    _check(load().mis_score_labels(ctypes.byref(seg.struct), _dev(hidden, "hidden"), H,
                                   _dev(lm_head, "lm_head"), V, _dtype_code(hidden),
                                   _ptr_i32(lab), K, 1 if apply_softmax else 0,
                                   _dev(scores, "scores"), _dev(ws, "ws"),
                                   ws.numel() * ws.element_size(), _stream(stream)))
    return scores


def mis_score_labels_noalloc(seg: Segments, hidden, lm_head, label_ids: Sequence[int],
                             apply_softmax: bool = False, scores=None, stream=None):
    """``mis_score_labels`` with the library's own per-GPU scratch instead of a
    workspace (the C call allocates nothing; pass ``scores`` to allocate
    nothing here either). Calls that overlap on one GPU race."""
    torch = _torch()
    if hidden.dim() != 2 or lm_head.dim() != 2 or hidden.shape[1] != lm_head.shape[1]:
        raise ValueError("hidden must be [T, H] and lm_head [V, H]")
    if hidden.shape[0] != seg.total_tokens:
        raise ValueError("hidden rows differ from the segments' token count")
    if hidden.dtype != lm_head.dtype:
        raise ValueError("hidden and lm_head dtypes differ")
    lab = _host_i32(label_ids)
    N, K = seg.total_items, len(lab)
    if scores is None:
        scores = torch.empty((N, K), dtype=torch.float32, device=hidden.device)
    elif scores.dtype != torch.float32 or tuple(scores.shape) != (N, K):
        raise ValueError("scores must be float32 [N, K]")
    _check(load().mis_score_labels_noalloc(ctypes.byref(seg.struct), _dev(hidden, "hidden"), hidden.shape[1],
                                           _dev(lm_head, "lm_head"), lm_head.shape[0], _dtype_code(hidden),
                                           _ptr_i32(lab), K, 1 if apply_softmax else 0, _dev(scores, "scores"),
                                           _stream(stream)))
    return scores


def mis_score_labels_at(positions, hidden, lm_head, label_ids: Sequence[int], apply_softmax: bool = False,
                        scores=None, ws=None, stream=None):
    """Label scores ``[R, K]`` (float32) at the token rows ``positions`` (host ints)."""
    torch = _torch()
    if hidden.dim() != 2 or lm_head.dim() != 2 or hidden.shape[1] != lm_head.shape[1]:
        raise ValueError("hidden must be [T, H] and lm_head [V, H]")
    if hidden.dtype != lm_head.dtype:
        raise ValueError("hidden and lm_head dtypes differ")
    pos = _host_i32(positions)
    lab = _host_i32(label_ids)
    R, K = len(pos), len(lab)
    H, V = hidden.shape[1], lm_head.shape[0]
    if scores is None:
        scores = torch.empty((R, K), dtype=torch.float32, device=hidden.device)
    elif scores.dtype != torch.float32 or tuple(scores.shape) != (R, K):
        raise ValueError("scores must be float32 [R, K]")
    if ws is None:
        nbytes = mis_score_workspace_bytes(R, V, max(K, 1), H, hidden.dtype) if K >= 1 else 256
        ws = torch.empty(nbytes, dtype=torch.uint8, device=hidden.device)
    _check(load().mis_score_labels_at(_ptr_i32(pos), R, hidden.shape[0], _dev(hidden, "hidden"), H,
                                      _dev(lm_head, "lm_head"), V, _dtype_code(hidden), _ptr_i32(lab), K,
                                      1 if apply_softmax else 0, _dev(scores, "scores"), _dev(ws, "ws"),
                                      ws.numel() * ws.element_size(), _stream(stream)))
    return scores
