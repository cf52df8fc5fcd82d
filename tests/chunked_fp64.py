"""fp64 chunk-wise KDA, written from the derivation the HIP kernels follow.

Test-only.  It exists to pin the chunked algebra (WY/UT form, 16-token tile
reference factoring, blocked forward substitution, and the split of the
output into a state-free intra term plus a state term) against the token
loop of the oracle, before any kernel is trusted.  It shares no code with the
HIP library.

Notation, one head of one sequence, chunk of C tokens starting from state S:
  Gam_t  = sum of g_s for s <= t inside the chunk (per channel)
  r_I    = Gam just before 16-token tile I (zero for the first tile)
  A_ts   = beta_t * sum_c k_t[c] k_s[c] exp(Gam_t[c] - Gam_s[c])      (s < t)
  P_ts   = sum_c q_t[c] k_s[c] exp(Gam_t[c] - Gam_s[c])               (s <= t)
  L^-1   = (I + A)^-1
  W      = L^-1 (beta * k * exp(Gam)),   Ut = L^-1 (beta * v)
  U      = Ut - W S
  O      = (q * exp(Gam)) S + P U
  S_next = Diag(exp(Gam_C)) S + (k * exp(Gam_C - Gam))^T U
Within tile pair (I, J <= I) the decay is factored as
  exp(Gam_t - Gam_s) = exp(Gam_t - r_I) * exp(r_I - Gam_s),
the first factor <= 1 and the second <= exp(80) on the diagonal tile because
a 16-token tile sums at least 16 * (-5) = -80 of log-decay (Kimi K3 blog
post, section on the lower bound on the log-decay).
"""
import numpy as np

TILE = 16


def unit_lower_inverse_blocked(A, tile=TILE):
    """(I + A)^-1 for strictly lower-triangular A by blocked forward
    substitution: each diagonal block row by row, then the off-diagonal blocks
    X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ."""
    n = A.shape[0]
    nb = n // tile
    X = np.zeros_like(A)
    for b in range(nb):
        s = slice(b * tile, (b + 1) * tile)
        Ab = A[s, s]
        Xb = np.zeros((tile, tile))
        for i in range(tile):
            row = np.zeros(tile)
            row[i] = 1.0
            for j in range(i):
                row -= Ab[i, j] * Xb[j]
            Xb[i] = row
        X[s, s] = Xb
    for d in range(1, nb):
        for I in range(d, nb):
            J = I - d
            si, sj = slice(I * tile, (I + 1) * tile), slice(J * tile, (J + 1) * tile)
            acc = np.zeros((tile, tile))
            for K in range(J, I):
                sk = slice(K * tile, (K + 1) * tile)
                acc += A[si, sk] @ X[sk, sj]
            X[si, sj] = -X[si, si] @ acc
    return X


def chunk_step(q, k, v, g, beta, S, *, split_output=False):
    """One chunk.  q, k, g: [C, dk]; v: [C, dv]; beta: [C]; S: [dk, dv].
    C must be a multiple of 16 (callers pad with neutral tokens).
    Returns (O [C, dv], S_next)."""
    C, dk = k.shape
    nt = C // TILE
    Gam = np.cumsum(g, axis=0)
    r = np.zeros((nt, dk))
    for I in range(1, nt):
        r[I] = Gam[I * TILE - 1]
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for I in range(nt):
        ri = slice(I * TILE, (I + 1) * TILE)
        Kp = k[ri] * np.exp(Gam[ri] - r[I])
        Qp = q[ri] * np.exp(Gam[ri] - r[I])
        for J in range(I + 1):
            rj = slice(J * TILE, (J + 1) * TILE)
            Km = k[rj] * np.exp(r[I] - Gam[rj])
            A[ri, rj] = Kp @ Km.T
            P[ri, rj] = Qp @ Km.T
    A = beta[:, None] * np.tril(A, -1)
    P = np.tril(P, 0)
    Linv = unit_lower_inverse_blocked(A)
    W = Linv @ (beta[:, None] * k * np.exp(Gam))
    Ut = Linv @ (beta[:, None] * v)
    QG = q * np.exp(Gam)
    Kt = k * np.exp(Gam[-1] - Gam)
    if split_output:
        # state-free part computed once per chunk, then one product with S
        Qprime = QG - P @ W
        Ointra = P @ Ut
        O = Ointra + Qprime @ S
        U = Ut - W @ S
    else:
        U = Ut - W @ S
        O = QG @ S + P @ U
    S_next = np.exp(Gam[-1])[:, None] * S + Kt.T @ U
    return O, S_next


def chunked_prefill(q, k, v, g, beta, h0=None, cu_seqlens=None, *, chunk=64,
                    split_output=False):
    """Chunk-wise KDA over packed [T, H, d] inputs (fp64).  Chunks restart at
    each sequence start; the tail chunk is padded with neutral tokens
    (g = 0, beta = 0, q = k = v = 0)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            for t0 in range(cu[n], cu[n + 1], chunk):
                L = min(chunk, cu[n + 1] - t0)
                pad = lambda a, w: np.concatenate([a, np.zeros((chunk - L,) + a.shape[1:])])
                sl = slice(t0, t0 + L)
                O, S = chunk_step(pad(q[sl, h], 0), pad(k[sl, h], 0), pad(v[sl, h], 0),
                                  pad(g[sl, h], 0), pad(beta[sl, h], 0), S,
                                  split_output=split_output)
                o[sl, h] = O[:L]
            ht[n, h] = S
    return o, ht
