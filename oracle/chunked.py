"""FP64 chunked WY forward + ReWY backward -- TEST INFRASTRUCTURE ONLY.

A second evaluation of the operator, independent of the token recurrence in
``rewy_oracle.c``: it follows the chunk algebra of the ReWY paper and is the
plain statement of what each chunk-level GPU stage computes.  numpy primitives
(matmul, triangular inverse via ``np.linalg.solve``) are its only building
blocks.  Notation, for one chunk of n rows and one head (paper, section
"The chunk system and conventional WY backward" and Appendix A):

    G   in-chunk cumulative natural-log decay, gamma = exp(G)    [n, K]
    E = beta * gamma * K,   Y = K / gamma,   Z = beta * V,   Qg = s * Q * gamma
    L = tril_strict(E Y^T),   Cq = tril_incl(Qg Y^T),   M = I + L,   A = M^{-1}
    W = A E,  U = A Z,  R = U - W S,  O = Qg S + Cq R
    Lambda = diag(gamma_last),  F = Y Lambda,  S_next = Lambda S + F^T R

Backward (paper Algorithm 1 "ReWY local pullback", Appendix 7.2-7.3 and the
complete reverse order of Appendix 10), with S+ the adjoint of S_next:

    Rbar = Cq^T dO + F S+                      (both uses of R accumulated first)
    P    = A^T Rbar                            shared sensitivity
    D    = -tril_strict(P R^T)
    Hq   = tril_incl(dO R^T),  Fbar = R S+^T
    Qgbar = dO S^T + Hq Y
    Ebar  = -P S^T + D Y
    Ybar  = D^T E + Hq^T Qg + Fbar Lambda
    dS    = Qg^T dO + Lambda S+ - E^T P        (-E^T P supplied once)
    lambar = rowsum(S * S+) + colsum(Y * Fbar)
    dq = s gamma Qgbar,  dk = beta gamma Ebar + Ybar / gamma,  dv = beta P
    dbeta = <gamma K, Ebar> + <V, P>           (erase + write, undivided)
    Gbar = Qg Qgbar + E Ebar - Y Ybar,  Gbar_last += lambar * gamma_last
    dg = reverse in-chunk cumulative sum of Gbar (summed over K for a scalar gate)

gamma and 1/gamma are formed directly, so this evaluation is valid while the
in-chunk |G| stays below ~700 (FP64 range); the tests keep to that.
"""
from __future__ import annotations

import numpy as np


def _tril(x, strict):
    return np.tril(x, -1 if strict else 0)


def _partition(L, chunk):
    """Chunk lengths for one sequence of length L (int chunk size or explicit list)."""
    if isinstance(chunk, int):
        out = [chunk] * (L // chunk)
        if L % chunk:
            out.append(L % chunk)
        return out
    lens = list(chunk)
    if sum(lens) != L:
        raise ValueError("partition does not cover the sequence")
    return lens


def _chunk_fwd(Q, K, V, G, beta, S, scale):
    n = Q.shape[0]
    gam = np.exp(G)
    E = beta[:, None] * gam * K
    Y = K / gam
    Z = beta[:, None] * V
    Qg = scale * Q * gam
    L = _tril(E @ Y.T, True)
    Cq = _tril(Qg @ Y.T, False)
    A = np.linalg.solve(np.eye(n) + L, np.eye(n))
    W = A @ E
    U = A @ Z
    R = U - W @ S
    O = Qg @ S + Cq @ R
    lam = gam[-1]
    F = Y * lam
    S_next = lam[:, None] * S + F.T @ R
    ctx = dict(gam=gam, E=E, Y=Y, Z=Z, Qg=Qg, L=L, Cq=Cq, A=A, W=W, U=U, R=R, lam=lam, F=F,
               S=S.copy())
    return O, S_next, ctx


def _chunk_bwd(ctx, Q, K, V, beta, dO, Splus, scale, scalar_gate, route, round_DH=None):
    gam, E, Y, Qg, Cq, A, R, lam, F, S, W, Z = (ctx[x] for x in
                                                ("gam", "E", "Y", "Qg", "Cq", "A", "R", "lam",
                                                 "F", "S", "W", "Z"))
    Rbar = Cq.T @ dO + F @ Splus
    if route == "expanded":
        # conventional seven-product WY graph (paper section 2), used to check that
        # ReWY reaches the same coefficient and input adjoints
        Wbar = -Rbar @ S.T
        Abar = Rbar @ Z.T + Wbar @ E.T
        D = _tril(-A.T @ Abar @ A.T, True)
        P = A.T @ Rbar
        Edir = A.T @ Wbar
    else:
        P = A.T @ Rbar
        D = -_tril(P @ R.T, True)
        Edir = -P @ S.T
    Hq = _tril(dO @ R.T, False)
    if round_DH is not None:  # operand-format experiment: D and Hq enter their products rounded
        D, Hq = round_DH(D), round_DH(Hq)
    Fbar = R @ Splus.T
    Qgbar = dO @ S.T + Hq @ Y
    Ebar = Edir + D @ Y
    Ybar = D.T @ E + Hq.T @ Qg + Fbar * lam
    dS = Qg.T @ dO + lam[:, None] * Splus - E.T @ P
    lambar = (S * Splus).sum(1) + (Y * Fbar).sum(0)
    dq = scale * gam * Qgbar
    dk = beta[:, None] * gam * Ebar + Ybar / gam
    dv = beta[:, None] * P
    dbeta = ((gam * K) * Ebar).sum(1) + (V * P).sum(1)
    Gbar = Qg * Qgbar + E * Ebar - Y * Ybar
    if scalar_gate and route in ("gram_eliminated", "gram_matrix"):
        # scalar gate: replace the D-parts of E*Ebar and Y*Ybar (their feature sums)
        # by the Gram-free reductions of paper section 3.4 / Appendix 9, or by the
        # explicit key-Gram reductions they eliminate
        g1 = np.log(gam[:, 0])
        nonD = Qg * Qgbar + E * Edir - Y * (Hq.T @ Qg + Fbar * lam)
        if route == "gram_eliminated":
            Gam = D * np.exp(g1[:, None] - g1[None, :])
            AK = Gam @ K
            BK = Gam.T @ (beta[:, None] * K)
            gl = beta * (K * AK).sum(1) - (K * BK).sum(1)
        else:
            J = D * (E @ Y.T)
            gl = J.sum(1) - J.sum(0)
        Gsum = nonD.sum(1) + gl
        Gsum[-1] += (lambar * lam).sum()
        dg = np.cumsum(Gsum[::-1])[::-1]
    else:
        Gbar[-1] += lambar * lam
        dg = np.cumsum(Gbar[::-1], axis=0)[::-1]
        if scalar_gate:
            dg = dg.sum(1)
    inter = dict(Rbar=Rbar, P=P, D=D, Hq=Hq, Fbar=Fbar, Qgbar=Qgbar, Ebar=Ebar, Ybar=Ybar)
    return dq, dk, dv, dbeta, dg, dS, inter


def _seq_iter(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = list(np.asarray(cu_seqlens).reshape(-1))
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def forward_backward(q, k, v, g, beta, dO=None, *, scale, h0=None, dht=None, cu_seqlens=None,
                     chunk=64, route="rewy", round_DH=None):
    """Chunked evaluation of forward (and backward when dO is given).

    ``chunk`` is a chunk size or, for a single sequence, an explicit list of
    chunk lengths (a nonuniform partition).  ``route`` selects the backward
    graph: "rewy" (Algorithm 1), "expanded" (the seven-product WY graph),
    "gram_eliminated" or "gram_matrix" (scalar-gate log-gate reductions).
    ``round_DH`` (default None: exact) is applied to D and Hq of every chunk
    before they enter their products; it lets a test measure what a lower
    operand format for these two coefficient matrices does to the gradients
    (the paper's precision contract, section "Execution and numerical
    precision" and the precision-eligibility appendix).
    Returns a dict with o, ht and, with dO, dq, dk, dv, dg, dbeta, dh0.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, T, H, K = q.shape
    V = v.shape[-1]
    beta = np.asarray(beta, dtype=np.float64)
    if g is None:
        gk = np.zeros((B, T, H, K))
        scalar = False
        gate_shape = None
    else:
        g = np.asarray(g, dtype=np.float64)
        scalar = g.ndim == 3
        gate_shape = g.shape
        gk = np.broadcast_to(g[..., None], (B, T, H, K)) if scalar else g
    seqs = _seq_iter(B, T, cu_seqlens)
    N = len(seqs)
    o = np.zeros((B, T, H, V))
    ht = np.zeros((N, H, K, V))
    back = dO is not None
    if back:
        dO = np.asarray(dO, dtype=np.float64)
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        dbeta = np.zeros_like(beta)
        dg = None if g is None else np.zeros(gate_shape)
        dh0 = np.zeros((N, H, K, V))
    for n, (b, t0, t1) in enumerate(seqs):
        lens = _partition(t1 - t0, chunk)
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(int) + t0
        for h in range(H):
            S = np.zeros((K, V)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            ctxs = []
            for c in range(len(lens)):
                a, e = starts[c], starts[c + 1]
                G = np.cumsum(gk[b, a:e, h], axis=0)
                O, S_next, ctx = _chunk_fwd(q[b, a:e, h], k[b, a:e, h], v[b, a:e, h], G,
                                            beta[b, a:e, h], S, scale)
                o[b, a:e, h] = O
                ctxs.append(ctx)
                S = S_next
            ht[n, h] = S
            if not back:
                continue
            Splus = np.zeros((K, V)) if dht is None else np.array(dht[n, h], dtype=np.float64)
            for c in range(len(lens) - 1, -1, -1):
                a, e = starts[c], starts[c + 1]
                r = _chunk_bwd(ctxs[c], q[b, a:e, h], k[b, a:e, h], v[b, a:e, h],
                               beta[b, a:e, h], dO[b, a:e, h], Splus, scale, scalar, route,
                               round_DH)
                dq[b, a:e, h], dk[b, a:e, h], dv[b, a:e, h], dbeta[b, a:e, h] = r[:4]
                if dg is not None:
                    dg[b, a:e, h] = r[4]
                Splus = r[5]
            dh0[n, h] = Splus
    out = dict(o=o, ht=ht)
    if back:
        out.update(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)
    return out


def chunk_intermediates(q, k, v, g, beta, dO, S, Splus, *, scale):
    """Forward and backward intermediates of ONE chunk (single head, row-stacked
    [n, *] arrays, g [n, K] or [n] or None).  For checking identities only."""
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    n, K = q.shape
    if g is None:
        gk = np.zeros((n, K))
    else:
        g = np.asarray(g, dtype=np.float64)
        gk = np.broadcast_to(g[:, None], (n, K)) if g.ndim == 1 else g
    G = np.cumsum(gk, axis=0)
    O, S_next, ctx = _chunk_fwd(q, k, v, G, np.asarray(beta, dtype=np.float64), S, scale)
    res = {}
    for route in ("rewy", "expanded"):
        r = _chunk_bwd(ctx, q, k, v, np.asarray(beta, dtype=np.float64), dO, Splus, scale,
                       False, route)
        res[route] = r[6] | {"dS": r[5]}
    return ctx, res
