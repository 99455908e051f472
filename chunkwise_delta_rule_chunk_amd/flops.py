"""Algorithmic FLOP counts of the chunkwise delta-rule operator.

Convention: a multiply-add counts 2; a triangular product counts only the
triangle the method needs (inclusive n(n+1)/2 or strict n(n-1)/2 entries);
the unit-triangular inverse counts n^3/3; exp2 and elementwise work are not
counted.  Executed work that the method does not need (recomputation,
padding, dense triangles) is never added.  The products are the ones of the
chunk algebra in the ReWY paper (Appendix A forward, Algorithm 1 and
Appendix 10 backward).
"""
from __future__ import annotations


def _tri(n, strict):
    return n * (n - 1) // 2 if strict else n * (n + 1) // 2


def local_wy_expanded(n, dk, dv):
    """Seven-product local WY backward (ReWY paper, section 3.2 / Appendix 7.4)."""
    return 2 * n * dk * dv + 4 * n * n * dv + 4 * n * n * dk + 4 * n ** 3


def local_wy_rewy(n, dk, dv):
    """Three-product ReWY local pullback (same passages)."""
    return 2 * n * dk * dv + 4 * n * n * dv


def forward_chunk(n, K, V):
    """Scores, solve, WY form, state scan and output for one chunk-head of n rows."""
    f = 2 * K * _tri(n, True)          # L = tril_strict(E Y^T)
    f += 2 * K * _tri(n, False)        # Cq = tril_incl(Qg Y^T)
    f += n ** 3 // 3                   # A = (I + L)^-1
    f += 2 * K * _tri(n, False)        # W = A E
    f += 2 * V * _tri(n, False)        # U = A Z
    f += 2 * n * K * V * 2             # R = U - W S ; S' = Lambda S + F^T R
    f += 2 * n * K * V                 # Qg S
    f += 2 * V * _tri(n, False)        # Cq R
    return f


def recompute_chunk(n, K, V):
    """Forward work re-executed by the backward under the recompute policy
    (everything but the output): reported separately, never in the numerator."""
    return forward_chunk(n, K, V) - 2 * n * K * V - 2 * V * _tri(n, False)


def backward_chunk(n, K, V):
    """Reverse scan, ReWY producer and consumers for one chunk-head of n rows."""
    f = 2 * V * _tri(n, False)         # Cq^T dO
    f += 2 * n * K * V * 3             # F dh+ ; Qg^T dO ; W^T Rbar
    f += 2 * V * _tri(n, False)        # P = A^T Rbar
    f += 2 * V * _tri(n, True)         # D = -tril_strict(P R^T)
    f += 2 * V * _tri(n, False)        # Hq = tril_incl(dO R^T)
    f += 2 * n * K * V * 3             # dO S^T ; P S^T ; Fbar = R dh+^T
    f += 2 * K * _tri(n, True) * 2     # D Y ; D^T E
    f += 2 * K * _tri(n, False) * 2    # Hq Y ; Hq^T Qg
    return f


def chunk_lengths(seq_lengths, C=64):
    out = []
    for L in seq_lengths:
        out += [C] * (L // C) + ([L % C] if L % C else [])
    return out


def workload_flops(seq_lengths, H, K, V, C=64):
    """(forward, backward, recompute) algorithmic FLOPs of a whole call."""
    ns = chunk_lengths(seq_lengths, C)
    fw = sum(forward_chunk(n, K, V) for n in ns) * H
    bw = sum(backward_chunk(n, K, V) for n in ns) * H
    rc = sum(recompute_chunk(n, K, V) for n in ns) * H
    return fw, bw, rc


# ---- the same products split by the kernel that executes them --------------
# (prep: F2-F4; forward scan: F5-F6; reverse scan: B1; chunk backward: B2-B4)

def prep_chunk(n, K, V):
    """Scores, solve and WY form (the chunk-parallel forward preparation)."""
    f = 2 * K * _tri(n, True) + 2 * K * _tri(n, False)   # L, Cq
    f += n ** 3 // 3                                     # (I + L)^-1
    f += 2 * K * _tri(n, False) + 2 * V * _tri(n, False)  # W = A E, U = A Z
    return f


def fwd_scan_chunk(n, K, V):
    """State scan and output: R, S update, Qg S, Cq R."""
    return 2 * n * K * V * 3 + 2 * V * _tri(n, False)


def bwd_scan_chunk(n, K, V):
    """Reverse scan: Cq^T dO, F dh+, Qg^T dO, W^T Rbar."""
    return 2 * V * _tri(n, False) + 2 * n * K * V * 3


def bwd_chunk_chunk(n, K, V):
    """ReWY producer and consumers: P, D, Hq, the three state products and the
    four matrix-intra contractions."""
    return backward_chunk(n, K, V) - bwd_scan_chunk(n, K, V)


def bwd_producer_chunk(n, K, V):
    """The ReWY producer alone: P = A^T Rbar and D = -tril_strict(P R^T)."""
    return 2 * V * _tri(n, False) + 2 * V * _tri(n, True)


def bwd_consumers_chunk(n, K, V):
    """The consumers alone: Hq, the three state products, matrix intra."""
    return bwd_chunk_chunk(n, K, V) - bwd_producer_chunk(n, K, V)


def kernel_flops(stage, seq_lengths, H, K, V, C=64):
    """Algorithmic FLOPs one launch of `stage` performs for the method (work
    re-executed under the recompute policy is not counted: a recompute prep
    counts zero, the fused backward scans count the reverse scan only)."""
    ns = chunk_lengths(seq_lengths, C)
    per = {"prep_forward": prep_chunk, "fwd_scan": fwd_scan_chunk,
           "bwd_scan": bwd_scan_chunk, "bwd_chunk": bwd_chunk_chunk,
           "bwd_producer": bwd_producer_chunk, "bwd_consumers": bwd_consumers_chunk}.get(stage)
    if per is None:
        return 0
    return sum(per(n, K, V) for n in ns) * H
