"""KDA parity oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this
package; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Two independent implementations of the same plain definition (Kimi K3
architecture blog post, section "a lower bound that removed a GPU code
path": a fixed-size recurrent state that decays as it goes; section on the
serving stack: the state is updated serially and in place):

* ``prefill`` / ``decode_step``: the C fp64 token loop in ``kda_oracle.c``
  (OpenMP over independent (sequence, head) chains), loaded with ctypes.
* ``prefill_np`` / ``decode_step_np``: a numpy fp64 twin of the same loop,
  for tiny sizes, used to cross-check the C code.

Per token (decay first, erase, write, read after the update)::

    S <- Diag(exp(g_t)) S
    S <- S - beta_t k_t (k_t^T S)
    S <- S + beta_t k_t v_t^T
    o_t = S^T q_t
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

NO_ERASE = 1  # oracle-only ablation flag: gated linear attention (no erase term)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, fp64).  Returns the path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.kda_oracle_prefill.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i64p,
                                       i64, i64, i64, i64, ctypes.c_uint,
                                       f64p, f64p, ctypes.c_int]
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_decode_step.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                           i64, i64, i64, i64, f64p, ctypes.c_int]
    lib.kda_oracle_decode_step.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, g, beta, h0=None, cu_seqlens=None, *, flags=0, nthreads=0):
    """fp64 token-loop KDA over packed sequences.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H, dk]; beta: [T, H] (any float
    dtype; converted to float32, which is exact for bf16 and fp32 inputs).
    A leading batch axis [B, T, ...] is accepted when cu_seqlens is None and
    treated as B sequences of length T.  h0: [N, H, dk, dv] or None.
    Returns (o [.., H, dv] fp64, ht [N, H, dk, dv] fp64).
    """
    q = np.asarray(q)
    batched = q.ndim == 4
    if batched:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs a packed [T, H, d] layout")
        B, T = q.shape[:2]
        flat = lambda a: np.asarray(a).reshape((B * T,) + np.asarray(a).shape[2:])
        q, k, v, g, beta = (flat(x) for x in (q, k, v, g, beta))
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        T = q.shape[0]
        cu = (np.array([0, T], dtype=np.int64) if cu_seqlens is None
              else np.asarray(cu_seqlens, dtype=np.int64))
    Tt, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != Tt:
        raise ValueError("cu_seqlens must start at 0 and end at T")
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    o = np.zeros((Tt, H, dv), dtype=np.float64)
    ht = np.zeros((N, H, dk, dv), dtype=np.float64)
    h0p = None
    if h0 is not None:
        h0a = np.ascontiguousarray(np.asarray(h0, dtype=np.float64)).reshape(N, H, dk, dv)
        h0p = _ptr(h0a, ctypes.c_double)
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    rc = _load().kda_oracle_prefill(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float), h0p,
        _ptr(cu, ctypes.c_int64), N, H, dk, dv, int(flags),
        _ptr(o, ctypes.c_double), _ptr(ht, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill rejected its arguments")
    if batched:
        o = o.reshape(B, T, H, dv)
    return o, ht


def decode_step(q, k, v, g, beta, state, *, nthreads=0):
    """One fp64 decode step for N sequences; ``state`` (fp64 [N,H,dk,dv]) is
    updated in place.  q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H].
    Returns o [N, H, dv] fp64."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        raise TypeError("state must be a C-contiguous float64 ndarray")
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_decode_step(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float),
        _ptr(state, ctypes.c_double), N, H, dk, dv, _ptr(o, ctypes.c_double),
        int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_decode_step rejected its arguments")
    return o


# --------------------------------------------------------------------------
# numpy fp64 twin of the same token loop (tiny sizes only)
# --------------------------------------------------------------------------

def _token_np(S, q, k, v, g, beta, erase=True):
    """One token for all heads at once.  S: [H, dk, dv] fp64 (updated)."""
    S *= np.exp(g)[:, :, None]                                   # decay
    if erase:
        kS = np.einsum("hc,hcj->hj", k, S)                        # k^T S
        S -= beta[:, None, None] * k[:, :, None] * kS[:, None, :]  # erase
    S += beta[:, None, None] * k[:, :, None] * v[:, None, :]       # write
    return np.einsum("hcj,hc->hj", S, q)                          # read


def prefill_np(q, k, v, g, beta, h0=None, cu_seqlens=None, *, erase=True):
    """numpy twin of ``prefill`` for packed [T, H, d] inputs."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    for n in range(N):
        S = (np.zeros((H, dk, dv)) if h0 is None
             else np.array(np.asarray(h0, dtype=np.float64)[n], copy=True))
        for t in range(cu[n], cu[n + 1]):
            o[t] = _token_np(S, q[t], k[t], v[t], g[t], beta[t], erase)
        ht[n] = S
    return o, ht


def decode_step_np(q, k, v, g, beta, state):
    """numpy twin of ``decode_step``: state [N, H, dk, dv] fp64, in place."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    o = np.zeros(q.shape[:2] + (v.shape[-1],))
    for n in range(q.shape[0]):
        o[n] = _token_np(state[n], q[n], k[n], v[n], g[n], beta[n])
    return o
