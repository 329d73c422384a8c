"""Python binding of libbsa: selector-driven block-sparse landmark attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP kernels of
libbsa.so (built in-tree by ``python -m block_sparse_attention_landmark_amd.build``).  PyTorch
provides device memory and the current HIP stream.  If the library is missing, every call
raises RuntimeError; there is no fallback path.

Entry points mirror the C ABI in include/bsa.h:

* ``pool_landmarks(k)``                           -> lm
* ``select_topk(q, lm, topk=..., seq_k=...)``      -> (idx, sc)
* ``attend_prefill(q, k, v, idx, sc, lm, mode)``  -> (out, lse)
* ``attend_decode(q, kc, vc, idx, sc, lm, mode)`` -> (out, lse)
* ``attend_prefill_backward(q, k, v, idx, sc, out, lse, dout, mode, lm)`` -> (dq, dk, dv, dsc, dlm)

* ``lsa_build_index(lm, seg_blocks, n_clusters)``  -> flat clustered index (dict of tensors)
* ``lsa_select(q, lm, index, topk=...)``          -> (idx, sc) from the clustered index

and ``prefill(q, k, v, ...)`` / ``decode(q, kc, vc, lm, ...)`` chain them (``prefill_lsa`` /
``decode_lsa`` with the clustered index in place of the per-block top-K).
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = [
    "MODES", "Params", "library_path", "load_library", "pool_landmarks", "select_topk",
    "attend_prefill", "attend_decode", "select_workspace_bytes", "decode_workspace_bytes",
    "prefill", "decode", "BsaError", "attend_prefill_backward", "backward_workspace_bytes",
    "lsa_build_index", "lsa_select", "prefill_lsa", "decode_lsa", "lsa_build_tree",
    "lsa_tree_select", "decode_step", "decode_step_paged", "decode_step_workspace_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
MODES = {"plain": 0, "sas": 1, "hils": 2}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_LIB = None


class BsaError(RuntimeError):
    """A non-zero status returned by libbsa."""

    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: status {status}: {detail}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seq_q", ctypes.c_int32), ("seq_k", ctypes.c_int32),
        ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("n_sink", ctypes.c_int32),
        ("n_local", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32),
    ]


def library_path() -> str:
    return os.path.join(_HERE, "libbsa.so")


def load_library():
    """Load libbsa.so (once).  Raises RuntimeError if it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = _open(library_path())
    return _LIB


@contextlib.contextmanager
def using_library(path: str):
    """Route every call made inside the block through another build of the library (the
    race-check build libbsa_sync.so, in the tests that compare the two builds' bits)."""
    global _LIB
    prev = load_library()
    _LIB = _open(path)
    try:
        yield _LIB
    finally:
        _LIB = prev


def _open(path: str):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_landmark_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Params)
    vp, st = ctypes.c_void_p, ctypes.c_int
    lib.bsa_pool_landmarks.argtypes = [P, vp, vp, vp]
    lib.bsa_pool_landmarks.restype = st
    lib.bsa_select_workspace_bytes.argtypes = [P]
    lib.bsa_select_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_select_topk.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bsa_select_topk.restype = st
    lib.bsa_select_topk_fused.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bsa_select_topk_fused.restype = st
    lib.bsa_attend_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_attend_prefill.restype = st
    lib.bsa_decode_workspace_bytes.argtypes = [P]
    lib.bsa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_attend_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bsa_attend_decode.restype = st
    i32 = ctypes.c_int32
    lib.bsa_pool_landmarks_paged.argtypes = [P, vp, i32, vp, vp, vp, vp]
    lib.bsa_pool_landmarks_paged.restype = st
    lib.bsa_select_topk_paged.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.bsa_select_topk_paged.restype = st
    lib.bsa_attend_decode_paged.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.c_size_t, vp]
    lib.bsa_attend_decode_paged.restype = st
    lib.bsa_decode_step_workspace_bytes.argtypes = [P]
    lib.bsa_decode_step_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_decode_step.argtypes = [P] + [vp] * 9 + [ctypes.c_size_t, vp]
    lib.bsa_decode_step.restype = st
    lib.bsa_decode_step_paged.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.c_size_t, vp]
    lib.bsa_decode_step_paged.restype = st
    lib.bsa_backward_workspace_bytes.argtypes = [P]
    lib.bsa_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_attend_prefill_backward.argtypes = [P] + [vp] * 15 + [ctypes.c_size_t, vp]
    lib.bsa_attend_prefill_backward.restype = st
    lib.bsa_lsa_build_index.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.bsa_lsa_build_index.restype = st
    lib.bsa_lsa_select_workspace_bytes.argtypes = [P]
    lib.bsa_lsa_select_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_lsa_select.argtypes = [P, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bsa_lsa_select.restype = st
    lib.bsa_lsa_tree_centres.argtypes = [P, vp, i32, i32, vp, vp, vp]
    lib.bsa_lsa_tree_centres.restype = st
    lib.bsa_lsa_tree_select.argtypes = [P, vp, vp, i32, i32, i32, i32] + [vp] * 7 + [vp, ctypes.c_size_t, vp]
    lib.bsa_lsa_tree_select.restype = st
    lib.bsa_update_landmarks.argtypes = [P, vp, i32, vp, vp]
    lib.bsa_update_landmarks.restype = st
    lib.bsa_update_landmarks_paged.argtypes = [P, vp, i32, vp, vp, i32, vp, vp]
    lib.bsa_update_landmarks_paged.restype = st
    lib.bsa_lsa_update_index.argtypes = [P, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.bsa_lsa_update_index.restype = st
    lib.bsa_attend_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_attend_decode_noalloc.restype = st
    lib.bsa_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.bsa_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_status_string.argtypes = [ctypes.c_int]
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_last_error.argtypes = []
    lib.bsa_last_error.restype = ctypes.c_char_p
    lib.bsa_version.argtypes = []
    lib.bsa_version.restype = ctypes.c_int
    return lib


def _check(fn: str, status: int):
    if status != 0:
        lib = load_library()
        raise BsaError(fn, status, f"{lib.bsa_status_string(status).decode()}: "
                                   f"{lib.bsa_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, shape=None):
    """Type, dtype, rank, exact shape and contiguity of a tensor handed to the library.  The
    C ABI receives bare pointers, so this is the only place where a buffer that is too small
    or of the wrong type can be caught.  The device is checked separately (_on_device), after
    every tensor of the call has passed this check."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(ref: torch.Tensor, **tensors):
    """Every tensor of a call lives on the same HIP device as `ref` (None entries skipped)."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a HIP device (got {ref.device})")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def make_params(*, B, Hq, Hkv, D, seq_q, seq_k, dtype, topk=0, n_sink=1, n_local=2, scale=0.0,
                mode="plain") -> Params:
    return Params(B, Hq, Hkv, D, seq_q, seq_k, 64, topk, n_sink, n_local, float(scale),
                  _DTYPES[dtype], MODES[mode] if isinstance(mode, str) else int(mode))


def _nblocks(T):
    return (T + 63) // 64


# ---------------------------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------------------------

def pool_landmarks(k: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """k [B,Hkv,T,D] -> landmarks [B,Hkv,ceil(T/64),D] (block means, rounded to k's dtype)."""
    lib = load_library()
    _need(k, "k", ndim=4)
    B, Hkv, T, D = k.shape
    if out is None:
        out = torch.empty((B, Hkv, _nblocks(T), D), dtype=k.dtype, device=k.device)
    _need(out, "lm", dtype=k.dtype, shape=(B, Hkv, _nblocks(T), D))
    _on_device(k, lm=out)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=k.dtype)
    _check("bsa_pool_landmarks", lib.bsa_pool_landmarks(ctypes.byref(p), _ptr(k), _ptr(out),
                                                        _stream(k.device)))
    return out


def update_landmarks(k: torch.Tensor, lm: torch.Tensor, n_new: int) -> torch.Tensor:
    """Recompute, in place, the landmarks of the blocks holding the last n_new tokens of
    k [B,Hkv,T,D] (the blocks that changed when those tokens were appended); returns lm."""
    lib = load_library()
    _need(k, "k", ndim=4)
    B, Hkv, T, D = k.shape
    _need(lm, "lm", dtype=k.dtype, shape=(B, Hkv, _nblocks(T), D))
    if int(n_new) < 1:
        raise ValueError("n_new must be >= 1")
    _on_device(k, lm=lm)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=k.dtype)
    _check("bsa_update_landmarks", lib.bsa_update_landmarks(ctypes.byref(p), _ptr(k), int(n_new),
                                                            _ptr(lm), _stream(k.device)))
    return lm


def select_workspace_bytes(p: Params) -> int:
    return int(load_library().bsa_select_workspace_bytes(ctypes.byref(p)))


def decode_workspace_bytes(p: Params) -> int:
    return int(load_library().bsa_decode_workspace_bytes(ctypes.byref(p)))


def lsa_select_workspace_bytes(p: Params) -> int:
    return int(load_library().bsa_lsa_select_workspace_bytes(ctypes.byref(p)))


def select_topk(q: torch.Tensor, lm: torch.Tensor, *, topk: int, seq_k: int | None = None,
                n_sink: int = 1, n_local: int = 2, ws: torch.Tensor | None = None,
                idx: torch.Tensor | None = None, sc: torch.Tensor | None = None,
                one_pass: bool = False):
    """Attended block sets.

    Prefill: q [B,Hq,T,D], lm [B,Hkv,ceil(T/64),D] -> idx, sc [B,Hkv,ceil(T/64),NA].
    Decode:  q [B,Hq,1,D], lm of the seq_k cached keys -> idx, sc [B,Hkv,1,NA].
    one_pass=True calls bsa_select_topk_fused (bf16 prefill, topk <= 32) at any length.
    """
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(lm, "lm", dtype=q.dtype, ndim=4)
    B, Hq, Tq, D = q.shape
    Hkv = lm.shape[1]
    Tk = Tq if seq_k is None else int(seq_k)
    _need(lm, "lm", shape=(B, Hkv, _nblocks(Tk), D))
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=Tq, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local)
    R = 1 if (Tq == 1 and Tk != 1) else _nblocks(Tq)
    NA = n_sink + n_local + topk
    if idx is None:
        idx = torch.empty((B, Hkv, R, NA), dtype=torch.int32, device=q.device)
    if sc is None:
        sc = torch.empty((B, Hkv, R, NA), dtype=torch.float32, device=q.device)
    _need(idx, "idx", dtype=torch.int32, shape=(B, Hkv, R, NA))
    _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, R, NA))
    need = select_workspace_bytes(p)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, lm=lm, idx=idx, sc=sc, ws=ws)
    name = "bsa_select_topk_fused" if one_pass else "bsa_select_topk"
    _check(name, getattr(lib, name)(ctypes.byref(p), _ptr(q), _ptr(lm), _ptr(idx), _ptr(sc),
                                    _ptr(ws), ws.numel(), _stream(q.device)))
    return idx, sc


def attend_prefill(q, k, v, idx, sc=None, lm=None, *, mode="plain", topk=None, n_sink=1,
                   n_local=2, scale=0.0, want_lse=False, out=None, lse=None):
    """Block-sparse prefill attention; returns (out [B,Hq,T,D], lse [B,Hq,T] or None)."""
    lib = load_library()
    _need(q, "q", ndim=4)
    B, Hq, T, D = q.shape
    _need(k, "k", dtype=q.dtype, ndim=4)
    Hkv = k.shape[1]
    _need(k, "k", shape=(B, Hkv, T, D))
    _need(v, "v", dtype=q.dtype, shape=(B, Hkv, T, D))
    _need(idx, "idx", dtype=torch.int32, ndim=4)
    NA = idx.shape[-1]
    if topk is None:
        topk = NA - n_sink - n_local
    if NA != n_sink + n_local + topk:
        raise ValueError(f"idx has {NA} entries per row, the call needs n_sink + n_local + topk")
    _need(idx, "idx", shape=(B, Hkv, _nblocks(T), NA))
    if sc is not None:
        _need(sc, "sc", dtype=torch.float32, shape=idx.shape)
    if lm is not None:
        _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, _nblocks(T), D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq, T))
    _on_device(q, k=k, v=v, idx=idx, sc=sc, lm=lm, out=out, lse=lse)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    _check("bsa_attend_prefill",
           lib.bsa_attend_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lm), _ptr(idx),
                                  _ptr(sc), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def attend_decode(q, kc, vc, idx, sc=None, lm=None, *, mode="plain", topk=None, n_sink=1,
                  n_local=2, scale=0.0, want_lse=False, out=None, lse=None, ws=None):
    """Block-sparse decode attention of the token at position Tk-1; q [B,Hq,1,D]."""
    lib = load_library()
    _need(q, "q", ndim=4)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B,Hq,1,D]")
    _need(kc, "kc", dtype=q.dtype, ndim=4)
    Hkv, Tk = kc.shape[1], kc.shape[2]
    _need(kc, "kc", shape=(B, Hkv, Tk, D))
    _need(vc, "vc", dtype=q.dtype, shape=(B, Hkv, Tk, D))
    _need(idx, "idx", dtype=torch.int32, ndim=4)
    NA = idx.shape[-1]
    if topk is None:
        topk = NA - n_sink - n_local
    if NA != n_sink + n_local + topk:
        raise ValueError(f"idx has {NA} entries per row, the call needs n_sink + n_local + topk")
    _need(idx, "idx", shape=(B, Hkv, 1, NA))
    if sc is not None:
        _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, 1, NA))
    if lm is not None:
        _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, _nblocks(Tk), D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    need = decode_workspace_bytes(p)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, kc=kc, vc=vc, idx=idx, sc=sc, lm=lm, out=out, lse=lse, ws=ws)
    _check("bsa_attend_decode",
           lib.bsa_attend_decode(ctypes.byref(p), _ptr(q), _ptr(kc), _ptr(vc), _ptr(lm), _ptr(idx),
                                 _ptr(sc), _ptr(out), _ptr(lse), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(q.device)))
    return out, lse


def attend_decode_noalloc(q, kc, vc, idx, sc=None, lm=None, *, mode="plain", topk=None,
                          n_sink=1, n_local=2, scale=0.0, out=None, lse=None):
    """attend_decode without a workspace: the library keeps the split partial states in its
    static per-device scratch (4 MiB; larger needs are rejected).  For callers that cannot
    allocate, so `out` (and `lse`, when wanted) should be passed in; calls on one device must
    not overlap."""
    lib = load_library()
    _need(q, "q", ndim=4)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B,Hq,1,D]")
    _need(kc, "kc", dtype=q.dtype, ndim=4)
    Hkv, Tk = kc.shape[1], kc.shape[2]
    _need(kc, "kc", shape=(B, Hkv, Tk, D))
    _need(vc, "vc", dtype=q.dtype, shape=(B, Hkv, Tk, D))
    _need(idx, "idx", dtype=torch.int32, ndim=4)
    NA = idx.shape[-1]
    if topk is None:
        topk = NA - n_sink - n_local
    if NA != n_sink + n_local + topk:
        raise ValueError(f"idx has {NA} entries per row, the call needs n_sink + n_local + topk")
    _need(idx, "idx", shape=(B, Hkv, 1, NA))
    if sc is not None:
        _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, 1, NA))
    if lm is not None:
        _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, _nblocks(Tk), D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    _on_device(q, kc=kc, vc=vc, idx=idx, sc=sc, lm=lm, out=out, lse=lse)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    _check("bsa_attend_decode_noalloc",
           lib.bsa_attend_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(kc), _ptr(vc), _ptr(lm),
                                         _ptr(idx), _ptr(sc), _ptr(out), _ptr(lse),
                                         _stream(q.device)))
    return out, lse


def backward_workspace_bytes(p: Params) -> int:
    return int(load_library().bsa_backward_workspace_bytes(ctypes.byref(p)))


def attend_prefill_backward(q, k, v, idx, sc, out, lse, dout, *, mode="plain", lm=None, topk=None,
                            n_sink=1, n_local=2, scale=0.0, ws=None, dq=None, dk=None, dv=None,
                            dsc=None, dlm=None):
    """Gradients of bf16 prefill attention given the forward's out (and lse for PLAIN / SAS).

    Returns (dq [B,Hq,T,D], dk, dv [B,Hkv,T,D], dsc [B,Hkv,ceil(T/64),NA] float32, dlm): dsc is
    the gradient with respect to the selector scores through the SAS gates (zeros otherwise);
    dlm [B,Hkv,ceil(T/64),D] float32 is, for HiLS (which needs lm, the forward's landmarks), the
    gradient with respect to the landmarks through the retrieval scores, else None.
    """
    lib = load_library()
    _need(q, "q", dtype=torch.bfloat16, ndim=4)
    B, Hq, T, D = q.shape
    _need(k, "k", dtype=q.dtype, ndim=4)
    Hkv = k.shape[1]
    _need(k, "k", shape=(B, Hkv, T, D))
    _need(v, "v", dtype=q.dtype, shape=(B, Hkv, T, D))
    if out is not None:
        _need(out, "out", dtype=q.dtype, shape=q.shape)
    _need(dout, "dout", dtype=q.dtype, shape=q.shape)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq, T))
    _need(idx, "idx", dtype=torch.int32, ndim=4)
    NA = idx.shape[-1]
    if topk is None:
        topk = NA - n_sink - n_local
    if NA != n_sink + n_local + topk:
        raise ValueError(f"idx has {NA} entries per row, the call needs n_sink + n_local + topk")
    _need(idx, "idx", shape=(B, Hkv, _nblocks(T), NA))
    if sc is not None:
        _need(sc, "sc", dtype=torch.float32, shape=idx.shape)
    if lm is not None:
        _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, _nblocks(T), D))
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if dsc is None:
        dsc = torch.empty(idx.shape, dtype=torch.float32, device=q.device)
    if mode == "hils" and dlm is None:
        dlm = torch.empty((B, Hkv, _nblocks(T), D), dtype=torch.float32, device=q.device)
    _need(dq, "dq", dtype=q.dtype, shape=q.shape)
    _need(dk, "dk", dtype=q.dtype, shape=k.shape)
    _need(dv, "dv", dtype=q.dtype, shape=k.shape)
    _need(dsc, "dsc", dtype=torch.float32, shape=idx.shape)
    if dlm is not None:
        _need(dlm, "dlm", dtype=torch.float32, shape=(B, Hkv, _nblocks(T), D))
    need = backward_workspace_bytes(p)
    if need == 0:
        need = 256    # the call itself reports why the shape is rejected
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, k=k, v=v, idx=idx, sc=sc, out=out, lse=lse, dout=dout, lm=lm, dq=dq, dk=dk,
               dv=dv, dsc=dsc, dlm=dlm, ws=ws)
    _check("bsa_attend_prefill_backward",
           lib.bsa_attend_prefill_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lm),
                                           _ptr(idx), _ptr(sc), _ptr(out), _ptr(lse), _ptr(dout),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsc), _ptr(dlm),
                                           _ptr(ws), ws.numel(), _stream(q.device)))
    return dq, dk, dv, dsc, (dlm if mode == "hils" else None)


def lsa_build_index(lm: torch.Tensor, *, seg_blocks: int = 64, n_clusters: int = 16) -> dict:
    """Flat clustered index of landmarks lm [B,Hkv,NB,D]: Ward clusters of every completed
    segment of seg_blocks landmarks.  Returns dict(centres [B,Hkv,NS*n_clusters,D] float32,
    members [B,Hkv,NS,seg_blocks] int32, offsets [B,Hkv,NS,n_clusters+1] int32,
    merges [B,Hkv,NS,seg_blocks-n_clusters,2] int32, seg_blocks, n_clusters), NS = NB // seg_blocks."""
    lib = load_library()
    _need(lm, "lm", ndim=4)
    B, Hkv, NB, D = lm.shape
    NS = NB // seg_blocks if seg_blocks > 0 else 0
    dev = lm.device
    centres = torch.empty((B, Hkv, NS * n_clusters, D), dtype=torch.float32, device=dev)
    members = torch.empty((B, Hkv, NS, seg_blocks), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, Hkv, NS, n_clusters + 1), dtype=torch.int32, device=dev)
    merges = torch.empty((B, Hkv, NS, max(seg_blocks - n_clusters, 0), 2), dtype=torch.int32,
                         device=dev)
    _on_device(lm)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=NB * 64, seq_k=NB * 64, dtype=lm.dtype)
    _check("bsa_lsa_build_index",
           lib.bsa_lsa_build_index(ctypes.byref(p), _ptr(lm), seg_blocks, n_clusters,
                                   _ptr(centres), _ptr(members), _ptr(offsets), _ptr(merges),
                                   _stream(dev)))
    return {"centres": centres, "members": members, "offsets": offsets, "merges": merges,
            "seg_blocks": seg_blocks, "n_clusters": n_clusters}


def _check_index(index: dict, B: int, Hkv: int, NB: int, D: int, tree: bool = False):
    """Shapes and dtypes of an index from lsa_build_index (and lsa_build_tree)."""
    seg, nc = int(index["seg_blocks"]), int(index["n_clusters"])
    if seg < 1:
        raise ValueError("index seg_blocks must be >= 1")
    NS = NB // seg
    _need(index["centres"], "centres", dtype=torch.float32, shape=(B, Hkv, NS * nc, D))
    _need(index["members"], "members", dtype=torch.int32, shape=(B, Hkv, NS, seg))
    _need(index["offsets"], "offsets", dtype=torch.int32, shape=(B, Hkv, NS, nc + 1))
    if tree:
        fan = int(index["fanout"])
        if fan < 1:
            raise ValueError("index fanout must be >= 1")
        _need(index["seg_centres"], "seg_centres", dtype=torch.float32, shape=(B, Hkv, NS, D))
        _need(index["grp_centres"], "grp_centres", dtype=torch.float32,
              shape=(B, Hkv, NS // fan, D))
    return NS


def _select_outputs(q, B, Hkv, R, NA, idx, sc):
    if idx is None:
        idx = torch.empty((B, Hkv, R, NA), dtype=torch.int32, device=q.device)
    if sc is None:
        sc = torch.empty((B, Hkv, R, NA), dtype=torch.float32, device=q.device)
    _need(idx, "idx", dtype=torch.int32, shape=(B, Hkv, R, NA))
    _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, R, NA))
    return idx, sc


def lsa_update_index(lm: torch.Tensor, index: dict, first_segment: int) -> dict:
    """Cluster, in place, only the segments first_segment .. NS-1 of an index from
    lsa_build_index (the segments completed since it was built up to first_segment); the
    clusters of earlier segments are kept as they are.  Returns the index."""
    lib = load_library()
    _need(lm, "lm", ndim=4)
    B, Hkv, NB, D = lm.shape
    _check_index(index, B, Hkv, NB, D)
    seg, nc = int(index["seg_blocks"]), int(index["n_clusters"])
    _need(index["merges"], "merges", dtype=torch.int32,
          shape=(B, Hkv, NB // seg, max(seg - nc, 0), 2))
    _on_device(lm, centres=index["centres"], members=index["members"],
               offsets=index["offsets"], merges=index["merges"])
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=NB * 64, seq_k=NB * 64, dtype=lm.dtype)
    _check("bsa_lsa_update_index",
           lib.bsa_lsa_update_index(ctypes.byref(p), _ptr(lm), seg, nc, int(first_segment),
                                    _ptr(index["centres"]), _ptr(index["members"]),
                                    _ptr(index["offsets"]), _ptr(index["merges"]),
                                    _stream(lm.device)))
    return index


def lsa_select(q: torch.Tensor, lm: torch.Tensor, index: dict, *, topk: int,
               seq_k: int | None = None, n_sink: int = 1, n_local: int = 2, ws=None, idx=None,
               sc=None):
    """Attended block sets from the flat clustered index (prefill: q [B,Hq,T,D]; decode:
    q [B,Hq,1,D] with seq_k cached tokens).  Same layout as select_topk's output."""
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(lm, "lm", dtype=q.dtype, ndim=4)
    B, Hq, Tq, D = q.shape
    Hkv = lm.shape[1]
    Tk = Tq if seq_k is None else int(seq_k)
    _need(lm, "lm", shape=(B, Hkv, _nblocks(Tk), D))
    NS = _check_index(index, B, Hkv, _nblocks(Tk), D)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=Tq, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local)
    R = 1 if (Tq == 1 and Tk != 1) else _nblocks(Tq)
    idx, sc = _select_outputs(q, B, Hkv, R, n_sink + n_local + topk, idx, sc)
    need = int(lib.bsa_lsa_select_workspace_bytes(ctypes.byref(p)))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    cen, mem, off = (index["centres"], index["members"], index["offsets"]) if NS else (None,) * 3
    _on_device(q, lm=lm, centres=cen, members=mem, offsets=off, idx=idx, sc=sc, ws=ws)
    _check("bsa_lsa_select",
           lib.bsa_lsa_select(ctypes.byref(p), _ptr(q), _ptr(lm), index["seg_blocks"],
                              index["n_clusters"], _ptr(cen), _ptr(mem), _ptr(off), _ptr(idx),
                              _ptr(sc), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(q.device)))
    return idx, sc


def lsa_build_tree(lm: torch.Tensor, index: dict, *, fanout: int = 8) -> dict:
    """Adds the tree's node centres to an index from lsa_build_index: seg_centres
    [B,Hkv,NS,D] and grp_centres [B,Hkv,NS // fanout,D] (float32); returns the index."""
    lib = load_library()
    _need(lm, "lm", ndim=4)
    B, Hkv, NB, D = lm.shape
    seg = index["seg_blocks"]
    if fanout < 1:
        raise ValueError("fanout must be >= 1")
    _check_index(index, B, Hkv, NB, D)
    NS = NB // seg
    seg_c = torch.empty((B, Hkv, NS, D), dtype=torch.float32, device=lm.device)
    grp_c = torch.empty((B, Hkv, NS // fanout, D), dtype=torch.float32, device=lm.device)
    _on_device(lm)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=NB * 64, seq_k=NB * 64, dtype=lm.dtype)
    _check("bsa_lsa_tree_centres",
           lib.bsa_lsa_tree_centres(ctypes.byref(p), _ptr(lm), seg, fanout, _ptr(seg_c),
                                    _ptr(grp_c), _stream(lm.device)))
    index.update(seg_centres=seg_c, grp_centres=grp_c, fanout=fanout)
    return index


def lsa_tree_select(q: torch.Tensor, lm: torch.Tensor, index: dict, *, topk: int, beam: int = 8,
                    seq_k: int | None = None, n_sink: int = 1, n_local: int = 2, ws=None,
                    idx=None, sc=None):
    """Attended block sets by beam search over the tree (index from lsa_build_index and
    lsa_build_tree); same layout as select_topk's output."""
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(lm, "lm", dtype=q.dtype, ndim=4)
    B, Hq, Tq, D = q.shape
    Hkv = lm.shape[1]
    Tk = Tq if seq_k is None else int(seq_k)
    _need(lm, "lm", shape=(B, Hkv, _nblocks(Tk), D))
    NS = _check_index(index, B, Hkv, _nblocks(Tk), D, tree=True)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=Tq, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local)
    R = 1 if (Tq == 1 and Tk != 1) else _nblocks(Tq)
    idx, sc = _select_outputs(q, B, Hkv, R, n_sink + n_local + topk, idx, sc)
    need = int(lib.bsa_lsa_select_workspace_bytes(ctypes.byref(p)))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    tens = [index[k] if NS else None for k in ("centres", "members", "offsets", "seg_centres")]
    grp = index["grp_centres"] if index["grp_centres"].shape[2] else None
    _on_device(q, lm=lm, centres=tens[0], members=tens[1], offsets=tens[2], seg_centres=tens[3],
               grp_centres=grp, idx=idx, sc=sc, ws=ws)
    _check("bsa_lsa_tree_select",
           lib.bsa_lsa_tree_select(ctypes.byref(p), _ptr(q), _ptr(lm), index["seg_blocks"],
                                   index["n_clusters"], index["fanout"], beam,
                                   *[_ptr(t) for t in tens], _ptr(grp), _ptr(idx), _ptr(sc),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(q.device)))
    return idx, sc


# ---------------------------------------------------------------------------------------------
# whole path
# ---------------------------------------------------------------------------------------------

def prefill(q, k, v, *, topk: int, mode: str = "plain", n_sink: int = 1, n_local: int = 2,
            scale: float = 0.0, want_lse: bool = False):
    """Pool, select and attend for a prefill; returns dict(out, lse, idx, sc, lm)."""
    lm = pool_landmarks(k)
    idx, sc = select_topk(q, lm, topk=topk, n_sink=n_sink, n_local=n_local)
    out, lse = attend_prefill(q, k, v, idx, sc, lm if mode == "hils" else None, mode=mode,
                              topk=topk, n_sink=n_sink, n_local=n_local, scale=scale,
                              want_lse=want_lse and mode != "hils")
    return {"out": out, "lse": lse, "idx": idx, "sc": sc, "lm": lm}


def decode(q, kc, vc, lm, *, topk: int, mode: str = "plain", n_sink: int = 1, n_local: int = 2,
           scale: float = 0.0, want_lse: bool = False):
    """Select and attend for one decode step (q [B,Hq,1,D]); returns dict(out, lse, idx, sc)."""
    idx, sc = select_topk(q, lm, topk=topk, seq_k=kc.shape[2], n_sink=n_sink, n_local=n_local)
    out, lse = attend_decode(q, kc, vc, idx, sc, lm if mode == "hils" else None, mode=mode,
                             topk=topk, n_sink=n_sink, n_local=n_local, scale=scale,
                             want_lse=want_lse and mode != "hils")
    return {"out": out, "lse": lse, "idx": idx, "sc": sc}


def decode_step_workspace_bytes(p: Params) -> int:
    return int(load_library().bsa_decode_step_workspace_bytes(ctypes.byref(p)))


def _step_outputs(q, B, Hkv, Hq, NA, idx, sc, out, lse, want_lse, mode):
    if idx is None:
        idx = torch.empty((B, Hkv, 1, NA), dtype=torch.int32, device=q.device)
    if sc is None:
        sc = torch.empty((B, Hkv, 1, NA), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and mode != "hils" and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(idx, "idx", dtype=torch.int32, shape=(B, Hkv, 1, NA))
    _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, 1, NA))
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    return idx, sc, out, lse


def decode_step(q, kc, vc, lm, *, topk: int, mode: str = "plain", n_sink: int = 1,
                n_local: int = 2, scale: float = 0.0, want_lse: bool = False, idx=None, sc=None,
                out=None, lse=None, ws=None):
    """One decode step (selection + attention) in one library call: q [B,Hq,1,D], kc/vc
    [B,Hkv,Tk,D], lm [B,Hkv,NB,D]; returns dict(out, lse, idx, sc) as decode() does."""
    lib = load_library()
    _need(q, "q", ndim=4)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B,Hq,1,D]")
    _need(kc, "kc", dtype=q.dtype, ndim=4)
    Hkv, Tk = kc.shape[1], kc.shape[2]
    _need(kc, "kc", shape=(B, Hkv, Tk, D))
    _need(vc, "vc", dtype=q.dtype, shape=(B, Hkv, Tk, D))
    _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, _nblocks(Tk), D))
    NA = n_sink + n_local + topk
    idx, sc, out, lse = _step_outputs(q, B, Hkv, Hq, NA, idx, sc, out, lse, want_lse, mode)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    need = decode_step_workspace_bytes(p)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, kc=kc, vc=vc, lm=lm, idx=idx, sc=sc, out=out, lse=lse, ws=ws)
    _check("bsa_decode_step",
           lib.bsa_decode_step(ctypes.byref(p), _ptr(q), _ptr(kc), _ptr(vc), _ptr(lm), _ptr(idx),
                               _ptr(sc), _ptr(out), _ptr(lse), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(q.device)))
    return {"out": out, "lse": lse, "idx": idx, "sc": sc}


# ---------------------------------------------------------------------------------------------
# paged (ragged) decode: 64-token pages [n_pages,Hkv,64,D], page_table [B,NB], seq_lens [B]
# ---------------------------------------------------------------------------------------------

def _paged_shapes(k_pool, page_table, seq_lens):
    _need(k_pool, "k_pool", ndim=4)
    _need(page_table, "page_table", dtype=torch.int32, ndim=2)
    n_pages, Hkv, blk, D = k_pool.shape
    if blk != 64:
        raise ValueError("k_pool must be [n_pages,Hkv,64,D]")
    B, NB = page_table.shape
    _need(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    return n_pages, Hkv, D, B, NB


def pool_landmarks_paged(k_pool, page_table, seq_lens, out=None):
    """Landmarks [B,Hkv,NB,D] of a paged cache (blocks past a sequence's end are zero)."""
    lib = load_library()
    n_pages, Hkv, D, B, NB = _paged_shapes(k_pool, page_table, seq_lens)
    if out is None:
        out = torch.empty((B, Hkv, NB, D), dtype=k_pool.dtype, device=k_pool.device)
    _need(out, "lm", dtype=k_pool.dtype, shape=(B, Hkv, NB, D))
    _on_device(k_pool, page_table=page_table, seq_lens=seq_lens, lm=out)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=NB * 64, seq_k=NB * 64, dtype=k_pool.dtype)
    _check("bsa_pool_landmarks_paged",
           lib.bsa_pool_landmarks_paged(ctypes.byref(p), _ptr(k_pool), int(n_pages),
                                        _ptr(page_table), _ptr(seq_lens), _ptr(out),
                                        _stream(k_pool.device)))
    return out


def update_landmarks_paged(k_pool, page_table, seq_lens, lm, n_new: int):
    """Recompute, in place, the landmarks [B,Hkv,NB,D] of the blocks holding each sequence's last
    n_new tokens (after appending n_new tokens to every sequence of a paged batch); returns lm."""
    lib = load_library()
    n_pages, Hkv, D, B, NB = _paged_shapes(k_pool, page_table, seq_lens)
    _need(lm, "lm", dtype=k_pool.dtype, shape=(B, Hkv, NB, D))
    if int(n_new) < 1:
        raise ValueError("n_new must be >= 1")
    _on_device(k_pool, page_table=page_table, seq_lens=seq_lens, lm=lm)
    p = make_params(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_q=NB * 64, seq_k=NB * 64, dtype=k_pool.dtype)
    _check("bsa_update_landmarks_paged",
           lib.bsa_update_landmarks_paged(ctypes.byref(p), _ptr(k_pool), int(n_pages),
                                          _ptr(page_table), _ptr(seq_lens), int(n_new), _ptr(lm),
                                          _stream(k_pool.device)))
    return lm


def select_topk_paged(q, lm, seq_lens, *, topk: int, n_sink: int = 1, n_local: int = 2,
                      idx=None, sc=None):
    """Attended sets of a paged decode batch: q [B,Hq,1,D], lm [B,Hkv,NB,D] -> idx, sc [B,Hkv,1,NA]."""
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(lm, "lm", dtype=q.dtype, ndim=4)
    B, Hq, one, D = q.shape
    Hkv, NB = lm.shape[1], lm.shape[2]
    if one != 1:
        raise ValueError("q must be [B,Hq,1,D]")
    _need(lm, "lm", shape=(B, Hkv, NB, D))
    _need(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    idx, sc = _select_outputs(q, B, Hkv, 1, n_sink + n_local + topk, idx, sc)
    _on_device(q, lm=lm, seq_lens=seq_lens, idx=idx, sc=sc)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=NB * 64, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local)
    _check("bsa_select_topk_paged",
           lib.bsa_select_topk_paged(ctypes.byref(p), _ptr(q), _ptr(lm), _ptr(seq_lens),
                                     _ptr(idx), _ptr(sc), _stream(q.device)))
    return idx, sc


def attend_decode_paged(q, k_pool, v_pool, page_table, seq_lens, idx, sc=None, lm=None, *,
                        mode="plain", topk=None, n_sink=1, n_local=2, scale=0.0, want_lse=False,
                        out=None, lse=None, ws=None):
    """Decode attention over a paged batch; q [B,Hq,1,D]; returns (out, lse or None)."""
    lib = load_library()
    _need(q, "q", ndim=4)
    n_pages, Hkv, D, B, NB = _paged_shapes(k_pool, page_table, seq_lens)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4)
    if v_pool.shape != k_pool.shape or k_pool.dtype != q.dtype:
        raise ValueError("v_pool must match k_pool, and both q's dtype")
    _need(idx, "idx", dtype=torch.int32, ndim=4)
    Hq = q.shape[1]
    _need(q, "q", shape=(B, Hq, 1, D))
    NA = idx.shape[-1]
    if topk is None:
        topk = NA - n_sink - n_local
    if NA != n_sink + n_local + topk:
        raise ValueError(f"idx has {NA} entries per row, the call needs n_sink + n_local + topk")
    _need(idx, "idx", shape=(B, Hkv, 1, NA))
    if sc is not None:
        _need(sc, "sc", dtype=torch.float32, shape=(B, Hkv, 1, NA))
    if lm is not None:
        _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, NB, D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=NB * 64, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    need = decode_workspace_bytes(p)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, k_pool=k_pool, v_pool=v_pool, page_table=page_table, seq_lens=seq_lens,
               idx=idx, sc=sc, lm=lm, out=out, lse=lse, ws=ws)
    _check("bsa_attend_decode_paged",
           lib.bsa_attend_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       int(n_pages), _ptr(page_table), _ptr(seq_lens), _ptr(lm),
                                       _ptr(idx), _ptr(sc), _ptr(out), _ptr(lse), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(q.device)))
    return out, lse


def decode_step_paged(q, k_pool, v_pool, page_table, seq_lens, lm, *, topk: int,
                      mode: str = "plain", n_sink: int = 1, n_local: int = 2, scale: float = 0.0,
                      want_lse: bool = False, idx=None, sc=None, out=None, lse=None, ws=None):
    """One paged decode step (selection + attention) in one library call; lm from
    pool_landmarks_paged; returns dict(out, lse, idx, sc)."""
    lib = load_library()
    _need(q, "q", ndim=4)
    n_pages, Hkv, D, B, NB = _paged_shapes(k_pool, page_table, seq_lens)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4)
    if v_pool.shape != k_pool.shape or k_pool.dtype != q.dtype:
        raise ValueError("v_pool must match k_pool, and both q's dtype")
    Hq = q.shape[1]
    _need(q, "q", shape=(B, Hq, 1, D))
    _need(lm, "lm", dtype=q.dtype, shape=(B, Hkv, NB, D))
    NA = n_sink + n_local + topk
    idx, sc, out, lse = _step_outputs(q, B, Hkv, Hq, NA, idx, sc, out, lse, want_lse, mode)
    p = make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=NB * 64, dtype=q.dtype, topk=topk,
                    n_sink=n_sink, n_local=n_local, scale=scale, mode=mode)
    need = decode_step_workspace_bytes(p)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, ndim=1)
    _on_device(q, k_pool=k_pool, v_pool=v_pool, page_table=page_table, seq_lens=seq_lens, lm=lm,
               idx=idx, sc=sc, out=out, lse=lse, ws=ws)
    _check("bsa_decode_step_paged",
           lib.bsa_decode_step_paged(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     int(n_pages), _ptr(page_table), _ptr(seq_lens), _ptr(lm),
                                     _ptr(idx), _ptr(sc), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(q.device)))
    return {"out": out, "lse": lse, "idx": idx, "sc": sc}


def decode_paged(q, k_pool, v_pool, page_table, seq_lens, *, topk: int, mode: str = "plain",
                 n_sink: int = 1, n_local: int = 2, scale: float = 0.0, want_lse: bool = False,
                 lm=None):
    """Pool (unless lm is given), select and attend for one paged decode step."""
    if lm is None:
        lm = pool_landmarks_paged(k_pool, page_table, seq_lens)
    idx, sc = select_topk_paged(q, lm, seq_lens, topk=topk, n_sink=n_sink, n_local=n_local)
    out, lse = attend_decode_paged(q, k_pool, v_pool, page_table, seq_lens, idx, sc,
                                   lm if mode == "hils" else None, mode=mode, topk=topk,
                                   n_sink=n_sink, n_local=n_local, scale=scale,
                                   want_lse=want_lse and mode != "hils")
    return {"out": out, "lse": lse, "idx": idx, "sc": sc, "lm": lm}


def prefill_lsa(q, k, v, *, topk: int, mode: str = "plain", seg_blocks: int = 64,
                n_clusters: int = 16, n_sink: int = 1, n_local: int = 2, scale: float = 0.0,
                want_lse: bool = False, tree: bool = False, fanout: int = 8, beam: int = 8):
    """Pool, build the clustered index, select from it (flat, or by beam search over the tree
    when tree=True) and attend, for a prefill; returns dict(out, lse, idx, sc, lm, index)."""
    lm = pool_landmarks(k)
    index = lsa_build_index(lm, seg_blocks=seg_blocks, n_clusters=n_clusters)
    if tree:
        lsa_build_tree(lm, index, fanout=fanout)
        idx, sc = lsa_tree_select(q, lm, index, topk=topk, beam=beam, n_sink=n_sink,
                                  n_local=n_local)
    else:
        idx, sc = lsa_select(q, lm, index, topk=topk, n_sink=n_sink, n_local=n_local)
    out, lse = attend_prefill(q, k, v, idx, sc, lm if mode == "hils" else None, mode=mode,
                              topk=topk, n_sink=n_sink, n_local=n_local, scale=scale,
                              want_lse=want_lse and mode != "hils")
    return {"out": out, "lse": lse, "idx": idx, "sc": sc, "lm": lm, "index": index}


def decode_lsa(q, kc, vc, lm, index, *, topk: int, mode: str = "plain", n_sink: int = 1,
               n_local: int = 2, scale: float = 0.0, want_lse: bool = False):
    """Select from the flat clustered index and attend, for one decode step (q [B,Hq,1,D])."""
    idx, sc = lsa_select(q, lm, index, topk=topk, seq_k=kc.shape[2], n_sink=n_sink,
                         n_local=n_local)
    out, lse = attend_decode(q, kc, vc, idx, sc, lm if mode == "hils" else None, mode=mode,
                             topk=topk, n_sink=n_sink, n_local=n_local, scale=scale,
                             want_lse=want_lse and mode != "hils")
    return {"out": out, "lse": lse, "idx": idx, "sc": sc}
