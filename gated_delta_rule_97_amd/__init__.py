"""Python binding of the MI355X Kimi Delta Attention library (libkda.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/kda.h``.  PyTorch supplies
device memory and the current stream; nothing here computes KDA.

Low-level functions carry the C names (``kda_chunk_prefill``,
``kda_chunk_prefill_noalloc``, ``kda_decode_step``, ``kda_chunk_prefill_workspace_size``,
``kda_status_string``, ``kda_profile_start``, ``kda_profile_stop``) and take
raw integer device addresses.  ``chunk_prefill`` and ``decode_step`` wrap
them for torch tensors.

Importing this package raises if the library has not been built
(``python gated_delta_rule_97_amd/build.py``): there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python gated_delta_rule_97_amd/build.py` (no CPU fallback exists)")

# A process must hold a single HIP runtime.  torch carries its own copy of
# libamdhip64 (same SONAME as the system one); loading torch before libkda.so
# makes the dynamic linker bind libkda.so to that copy.  Loaded the other way
# round, torch would map a second runtime next to the first.
try:
    import torch as _torch_mod  # noqa: F401
except ImportError:  # a plain C-ABI user without torch
    _torch_mod = None

_lib = ctypes.CDLL(LIB_PATH)

KDA_OK = 0
KDA_ERR_NULL = -1
KDA_ERR_SHAPE = -2
KDA_ERR_UNSUPPORTED = -3
KDA_ERR_WORKSPACE = -4
KDA_ERR_ALIGN = -5
KDA_ERR_ALIAS = -6
KDA_ERR_LAUNCH = -7
KDA_ERR_DECAY_BOUND = -8
KDA_ERR_TOO_LARGE = -9
NOALLOC_SCRATCH_BYTES = 128 << 20
KDA_FLAG_CHECK_DECAY = 1
KDA_FLAG_NO_SEGMENTS = 2
KDA_FLAG_NO_WINDOWS = 4
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

_vp, _i, _u, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


_lib.kda_chunk_prefill_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)]
_lib.kda_chunk_prefill_workspace_size.restype = _i
_lib.kda_chunk_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _u,
                                   _vp, _vp, _vp, _sz, _vp]
_lib.kda_chunk_prefill.restype = _i
_lib.kda_chunk_prefill_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _u,
                                           _vp, _vp, _vp]
_lib.kda_chunk_prefill_noalloc.restype = _i
_lib.kda_chunk_prefill_checkpointed.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                                _i, _u, _vp, _vp, _vp, _i, _i, _vp, _sz, _vp]
_lib.kda_chunk_prefill_checkpointed.restype = _i
_lib.kda_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _u, _vp]
_lib.kda_decode_step.restype = _i
_lib.kda_decode_verify.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _u, _vp]
_lib.kda_decode_verify.restype = _i
_lib.kda_decode_commit.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _u, _vp]
_lib.kda_decode_commit.restype = _i
_lib.kda_decode_verify_keep.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _u, _vp]
_lib.kda_decode_verify_keep.restype = _i
_lib.kda_decode_commit_kept.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _u, _vp]
_lib.kda_decode_commit_kept.restype = _i
_lib.kda_decode_commit_verify.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                          _i, _i, _i, _u, _vp]
_lib.kda_decode_commit_verify.restype = _i
_lib.kda_status_string.argtypes = [_i]
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_profile_start.argtypes = [_i]
_lib.kda_profile_start.restype = _i
_lib.kda_profile_stop.argtypes = [ctypes.POINTER(KernelTime), _i, ctypes.POINTER(_i)]
_lib.kda_profile_stop.restype = _i


class KdaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: status {status} ({kda_status_string(status)})")


# ----------------------------------------------------------- C-name wrappers

def kda_status_string(status: int) -> str:
    return _lib.kda_status_string(int(status)).decode()


def kda_chunk_prefill_workspace_size(B, T, H, dk, dv, num_seqs, chunk_size, dtype) -> int:
    n = _sz(0)
    st = _lib.kda_chunk_prefill_workspace_size(B, T, H, dk, dv, num_seqs, chunk_size, dtype, ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_prefill_workspace_size")
    return int(n.value)


def kda_chunk_prefill(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size, dtype,
                      flags, o, ht, workspace, workspace_bytes, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_chunk_prefill(q or None, k or None, v or None, g or None, beta or None, h0 or None,
                                  cu_seqlens or None, B, T, H, dk, dv, num_seqs, chunk_size, dtype, flags,
                                  o or None, ht or None, workspace or None, workspace_bytes, stream or None)


def kda_chunk_prefill_noalloc(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size, dtype,
                              flags, o, ht, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_chunk_prefill_noalloc(q or None, k or None, v or None, g or None, beta or None, h0 or None,
                                          cu_seqlens or None, B, T, H, dk, dv, num_seqs, chunk_size, dtype, flags,
                                          o or None, ht or None, stream or None)


def kda_chunk_prefill_checkpointed(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size,
                                   dtype, flags, o, ht, ckpt, ckpt_stride, num_ckpt, workspace, workspace_bytes,
                                   stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_chunk_prefill_checkpointed(q or None, k or None, v or None, g or None, beta or None,
                                               h0 or None, cu_seqlens or None, B, T, H, dk, dv, num_seqs,
                                               chunk_size, dtype, flags, o or None, ht or None, ckpt or None,
                                               ckpt_stride, num_ckpt, workspace or None, workspace_bytes,
                                               stream or None)


def kda_decode_step(q, k, v, g, beta, state, o, N, H, dk, dv, dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_step(q or None, k or None, v or None, g or None, beta or None, state or None,
                                o or None, N, H, dk, dv, dtype, flags, stream or None)


def kda_decode_verify(q, k, v, g, beta, state, o, N, K, H, dk, dv, dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_verify(q or None, k or None, v or None, g or None, beta or None, state or None,
                                  o or None, N, K, H, dk, dv, dtype, flags, stream or None)


def kda_decode_commit(k, v, g, beta, n_accept, state, N, K, H, dk, dv, dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_commit(k or None, v or None, g or None, beta or None, n_accept or None,
                                  state or None, N, K, H, dk, dv, dtype, flags, stream or None)


def kda_decode_verify_keep(q, k, v, g, beta, state, o, u, N, K, H, dk, dv, dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_verify_keep(q or None, k or None, v or None, g or None, beta or None, state or None,
                                       o or None, u or None, N, K, H, dk, dv, dtype, flags, stream or None)


def kda_decode_commit_kept(k, g, u, n_accept, state, N, K, H, dk, dv, dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_commit_kept(k or None, g or None, u or None, n_accept or None, state or None, N, K, H,
                                       dk, dv, dtype, flags, stream or None)


def kda_decode_commit_verify(prev_k, prev_g, prev_u, n_accept, Kp, q, k, v, g, beta, state, o, u, N, K, H, dk, dv,
                             dtype, flags, stream) -> int:
    """Raw call; pointers are ints (0 = NULL).  Returns the status code."""
    return _lib.kda_decode_commit_verify(prev_k or None, prev_g or None, prev_u or None, n_accept or None, Kp,
                                         q or None, k or None, v or None, g or None, beta or None, state or None,
                                         o or None, u or None, N, K, H, dk, dv, dtype, flags, stream or None)


def kda_profile_start(max_launches: int) -> None:
    st = _lib.kda_profile_start(int(max_launches))
    if st != KDA_OK:
        raise KdaError(st, "kda_profile_start")


def kda_profile_stop() -> dict:
    """Returns {kernel name: (launches, total_ms)} for the closed session."""
    buf = (KernelTime * 64)()
    n = _i(0)
    st = _lib.kda_profile_stop(buf, 64, ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_profile_stop")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, 64))}


# ------------------------------------------------------------ torch wrappers

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shapes(*checks):
    """Every given tensor has the shape the sizes passed to the library
    imply: (tensor or None, expected shape, name); a None entry in the
    expected shape matches any extent.  Checked before anything is launched,
    so a mismatched tensor is an error here rather than an out-of-bounds
    access on the device."""
    for t, shape, name in checks:
        if t is None:
            continue
        got = tuple(t.shape)
        if len(got) != len(shape) or any(e is not None and g != e for g, e in zip(got, shape)):
            want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
            raise ValueError(f"{name} has shape {list(got)}, expected {want}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_bytes(B, T, H, dk, dv, num_seqs, chunk_size, dtype) -> int:
    return kda_chunk_prefill_workspace_size(B, T, H, dk, dv, num_seqs, chunk_size, dtype)


def checkpoint_count(T, ckpt_stride, B=1, seqlens=None) -> int:
    """Checkpoint slots a checkpointed prefill writes: sum of len // stride
    over the sequences (B of length T, or the given lengths)."""
    if seqlens is not None:
        return int(sum(int(n) // ckpt_stride for n in seqlens))
    return int(B) * (int(T) // ckpt_stride)


def chunk_prefill(q, k, v, g, beta, h0=None, cu_seqlens=None, *, chunk_size=64, o=None, ht=None,
                  output_final_state=True, workspace=None, flags=0, stream=None, ckpt_stride=None, ckpt=None):
    """Chunked KDA prefill on device tensors.

    q, k [B, T, H, dk]; v [B, T, H, dv] (bf16 or fp32, same dtype);
    g [B, T, H, dk] fp32; beta [B, T, H] fp32; h0 [N, H, dk, dv] fp32 or None;
    cu_seqlens int32 [N+1] (packed, B = 1) or None.  Returns (o, ht).
    With ckpt_stride (a multiple of chunk_size) the call also writes strided
    state checkpoints and returns (o, ht, ckpt), ckpt [num_ckpt, H, dk, dv]
    fp32 (allocated from the sequence lengths when not given)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    _shapes((k, (B, T, H, dk), "k"), (v, (B, T, H, dv), "v"), (g, (B, T, H, dk), "g"), (beta, (B, T, H), "beta"),
            (h0, (N, H, dk, dv), "h0"), (o, (B, T, H, dv), "o"), (ht, (N, H, dk, dv), "ht"),
            (ckpt, (None, H, dk, dv), "ckpt"))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if ht is None and output_final_state:
        ht = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    need = workspace_bytes(B, T, H, dk, dv, N, chunk_size, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if ckpt_stride is not None:
        if ckpt is None:
            lens = None
            if cu_seqlens is not None:
                cu = cu_seqlens.cpu().tolist()
                lens = [cu[i + 1] - cu[i] for i in range(N)]
            ckpt = torch.empty((checkpoint_count(T, ckpt_stride, B, lens), H, dk, dv), dtype=torch.float32,
                               device=q.device)
        st = kda_chunk_prefill_checkpointed(
            _ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"), _ptr(g, torch.float32, "g"),
            _ptr(beta, torch.float32, "beta"), _ptr(h0, torch.float32, "h0"),
            _ptr(cu_seqlens, torch.int32, "cu_seqlens"), B, T, H, dk, dv, N, chunk_size, dt, flags,
            _ptr(o, q.dtype, "o"), _ptr(ht, torch.float32, "ht"), _ptr(ckpt, torch.float32, "ckpt"),
            int(ckpt_stride), ckpt.shape[0], _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
            _stream(stream))
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_prefill_checkpointed")
        return o, ht, ckpt
    st = kda_chunk_prefill(_ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"),
                           _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
                           _ptr(h0, torch.float32, "h0"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
                           B, T, H, dk, dv, N, chunk_size, dt, flags,
                           _ptr(o, q.dtype, "o"), _ptr(ht, torch.float32, "ht"),
                           _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_prefill")
    return o, ht


def decode_step(q, k, v, g, beta, state, o=None, *, flags=0, stream=None):
    """One decode step: q, k [N, H, dk]; v [N, H, dv]; g [N, H, dk] fp32;
    beta [N, H] fp32; state [N, H, dk, dv] fp32 updated in place.  Returns o."""
    torch = _torch()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    _shapes((k, (N, H, dk), "k"), (v, (N, H, dv), "v"), (g, (N, H, dk), "g"), (beta, (N, H), "beta"),
            (state, (N, H, dk, dv), "state"), (o, (N, H, dv), "o"))
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = kda_decode_step(_ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"),
                         _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
                         _ptr(state, torch.float32, "state"), _ptr(o, q.dtype, "o"),
                         N, H, dk, dv, dt, flags, _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o


def decode_verify(q, k, v, g, beta, state, o=None, *, keep_u=False, u=None, flags=0, stream=None):
    """K draft tokens per sequence from the committed state (left unchanged):
    q, k [N, K, H, dk]; v [N, K, H, dv]; g [N, K, H, dk] fp32; beta [N, K, H]
    fp32; state [N, H, dk, dv] fp32.  Returns o [N, K, H, dv]; with keep_u
    (or a u buffer given) also each draft's update vector u [N, K, H, dv]
    fp32, for decode_commit(..., u=u), and returns (o, u)."""
    torch = _torch()
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    _shapes((k, (N, K, H, dk), "k"), (v, (N, K, H, dv), "v"), (g, (N, K, H, dk), "g"), (beta, (N, K, H), "beta"),
            (state, (N, H, dk, dv), "state"), (o, (N, K, H, dv), "o"), (u, (N, K, H, dv), "u"))
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=q.dtype, device=q.device)
    keep = keep_u or u is not None
    if keep and u is None:
        u = torch.empty((N, K, H, dv), dtype=torch.float32, device=q.device)
    args = (_ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"), _ptr(g, torch.float32, "g"),
            _ptr(beta, torch.float32, "beta"), _ptr(state, torch.float32, "state"), _ptr(o, q.dtype, "o"))
    if keep:
        st = kda_decode_verify_keep(*args, _ptr(u, torch.float32, "u"), N, K, H, dk, dv, dt, flags, _stream(stream))
    else:
        st = kda_decode_verify(*args, N, K, H, dk, dv, dt, flags, _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_verify_keep" if keep else "kda_decode_verify")
    return (o, u) if keep else o


def decode_commit_verify(prev, q, k, v, g, beta, state, o=None, *, keep_u=True, u=None, flags=0, stream=None):
    """One round of a speculative loop in one pass over the states: commits
    the previous round's accepted drafts, prev = (k, g, u, n_accept) with u
    the update vectors that round's verify kept (None: nothing to commit),
    writes the committed state, and verifies the new drafts q, k, v, g, beta
    [N, K, H, .] from it.  Returns (o, u) with u the new drafts' update
    vectors for the next round (o only when keep_u is False and no u is
    given)."""
    torch = _torch()
    N, K, H, dk = q.shape
    dv = state.shape[-1]
    dt = _dtype_code(q)
    if prev is None:
        pk = pg = pu = pa = None
        Kp = 0
    else:
        pk, pg, pu, pa = prev
        Kp = pk.shape[1]
    _shapes((k, (N, K, H, dk), "k"), (v, (N, K, H, dv), "v"), (g, (N, K, H, dk), "g"), (beta, (N, K, H), "beta"),
            (state, (N, H, dk, dv), "state"), (o, (N, K, H, dv), "o"), (u, (N, K, H, dv), "u"),
            (pk, (N, Kp, H, dk), "prev k"), (pg, (N, Kp, H, dk), "prev g"), (pu, (N, Kp, H, dv), "prev u"),
            (pa, (N,), "n_accept"))
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=q.dtype, device=q.device)
    keep = keep_u or u is not None
    if keep and u is None:
        u = torch.empty((N, K, H, dv), dtype=torch.float32, device=q.device)
    st = kda_decode_commit_verify(_ptr(pk, q.dtype, "prev k"), _ptr(pg, torch.float32, "prev g"),
                                  _ptr(pu, torch.float32, "prev u"), _ptr(pa, torch.int32, "n_accept"), Kp,
                                  _ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"),
                                  _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
                                  _ptr(state, torch.float32, "state"), _ptr(o, q.dtype, "o"),
                                  _ptr(u, torch.float32, "u") if keep else 0, N, K, H, dk, dv, dt, flags,
                                  _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_commit_verify")
    return (o, u) if keep else o


def decode_commit(k, v, g, beta, n_accept, state, *, u=None, flags=0, stream=None):
    """Folds the first n_accept[n] (int32 [N] on the device) of the K draft
    tokens into each sequence's state, in place.  With u, the update vectors
    decode_verify kept on this same state and these drafts, the accepted
    drafts are applied in closed form from them (v and beta are then not
    read).  Returns state."""
    torch = _torch()
    N, K, H, dk = k.shape
    dv = state.shape[-1]
    dt = _dtype_code(k)
    _shapes((g, (N, K, H, dk), "g"), (n_accept, (N,), "n_accept"), (state, (N, H, dk, dv), "state"),
            (u, (N, K, H, dv), "u"))
    if u is None:
        _shapes((v, (N, K, H, dv), "v"), (beta, (N, K, H), "beta"))
    if u is not None:
        st = kda_decode_commit_kept(_ptr(k, k.dtype, "k"), _ptr(g, torch.float32, "g"), _ptr(u, torch.float32, "u"),
                                    _ptr(n_accept, torch.int32, "n_accept"), _ptr(state, torch.float32, "state"),
                                    N, K, H, dk, dv, dt, flags, _stream(stream))
        if st != KDA_OK:
            raise KdaError(st, "kda_decode_commit_kept")
        return state
    st = kda_decode_commit(_ptr(k, k.dtype, "k"), _ptr(v, k.dtype, "v"), _ptr(g, torch.float32, "g"),
                           _ptr(beta, torch.float32, "beta"), _ptr(n_accept, torch.int32, "n_accept"),
                           _ptr(state, torch.float32, "state"), N, K, H, dk, dv, dt, flags, _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_commit")
    return state
