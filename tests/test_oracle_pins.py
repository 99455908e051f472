"""Pins of the FP64 oracle to facts other than itself (CPU only).

Each test names the passage that fixes the expected value.  Together they are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
in either oracle evaluation fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunked

RNG = np.random.default_rng(12345)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(B, T, H, K, V, gate, seed, beta_range=(0.1, 0.9), gscale=0.3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, K))
    k = _unit(r.standard_normal((B, T, H, K)))
    v = r.standard_normal((B, T, H, V))
    beta = r.uniform(*beta_range, size=(B, T, H))
    if gate == "vector":
        g = -np.abs(r.standard_normal((B, T, H, K))) * gscale
    elif gate == "scalar":
        g = -np.abs(r.standard_normal((B, T, H))) * gscale
    else:
        g = None
    return q, k, v, g, beta


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_write_then_read(gate):
    """KDA blog section 2.1: with beta = 1 and a unit key, reading the state
    right after the write returns the written value exactly, for any decay."""
    T, K, V = 9, 6, 5
    q, k, v, g, _ = _inputs(1, T, 1, K, V, gate, 1)
    beta = np.ones((1, T, 1))
    h0 = RNG.standard_normal((1, 1, K, V))
    for t in range(T):
        sl = slice(0, t + 1)
        _, ht = oracle.forward(q[:, sl], k[:, sl], v[:, sl], None if g is None else g[:, sl],
                               beta[:, sl], scale=1.0, h0=h0)
        np.testing.assert_allclose(ht[0, 0].T @ k[0, t, 0], v[0, t, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("gate", ["none", "vector"])
def test_locality(gate):
    """KDA blog section 2.1: the rank-one write leaves every direction
    orthogonal to the current key unchanged: (S_t - S~_t)^T x = 0 for x _|_ k_t,
    where S~_t is the decayed previous state."""
    T, K, V = 7, 6, 4
    q, k, v, g, beta = _inputs(1, T, 1, K, V, gate, 2)
    h0 = RNG.standard_normal((1, 1, K, V))
    prev = h0[0, 0]
    for t in range(T):
        sl = slice(0, t + 1)
        _, ht = oracle.forward(q[:, sl], k[:, sl], v[:, sl], None if g is None else g[:, sl],
                               beta[:, sl], scale=1.0, h0=h0)
        a = np.ones(K) if g is None else np.exp(g[0, t, 0])
        St_dec = a[:, None] * prev
        x = RNG.standard_normal(K)
        kt = k[0, t, 0]
        x -= (x @ kt) * kt
        np.testing.assert_allclose((ht[0, 0] - St_dec).T @ x, 0.0, atol=1e-13)
        prev = ht[0, 0]


def test_linear_attention_reduction():
    """KDA blog section 1.1: with the erase gate 0, write gate 1 and no decay the
    recurrence is causal linear attention, o_t = s * sum_{j<=t} <k_j, q_t> v_j
    (+ s * S0^T q_t for an initial state); brute force O(T^2)."""
    B, T, H, K, V = 2, 23, 2, 5, 4
    q, k, v, _, _ = _inputs(B, T, H, K, V, "none", 3)
    h0 = RNG.standard_normal((B, H, K, V))
    s = 0.7
    o, ht = oracle.forward(q, k, v, None, None, scale=s, h0=h0,
                           erase=np.zeros((B, T, H, K)), write=np.ones((B, T, H, V)))
    ref = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = s * h0[b, h].T @ q[b, t, h]
                for j in range(t + 1):
                    acc = acc + s * (k[b, j, h] @ q[b, t, h]) * v[b, j, h]
                ref[b, t, h] = acc
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_gated_linear_attention_reduction():
    """Erase 0, write 1, vector decay: the decayed linear-attention form
    o_t = s * sum_{j<=t} <q_t * exp(G_t - G_j), k_j> v_j + s (exp(G_t) * q_t)^T S0
    with G the cumulative decay over the whole sequence (ReWY paper,
    Appendix A: a write at j is decayed by tokens j+1..t)."""
    B, T, H, K, V = 1, 19, 1, 4, 3
    q, k, v, g, _ = _inputs(B, T, H, K, V, "vector", 4)
    h0 = RNG.standard_normal((B, H, K, V))
    s = 0.5
    o, _ = oracle.forward(q, k, v, g, None, scale=s, h0=h0,
                          erase=np.zeros((B, T, H, K)), write=np.ones((B, T, H, V)))
    G = np.cumsum(g[0, :, 0], axis=0)
    for t in range(T):
        acc = s * (np.exp(G[t]) * q[0, t, 0]) @ h0[0, 0]
        for j in range(t + 1):
            acc = acc + s * ((q[0, t, 0] * np.exp(G[t] - G[j])) @ k[0, j, 0]) * v[0, j, 0]
        np.testing.assert_allclose(o[0, t, 0], acc, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_beta_zero_is_pure_decay(gate):
    """With beta = 0 nothing is written: S_t = diag(exp G_t) S0 and
    o_t = S_t^T (s q_t)."""
    B, T, H, K, V = 1, 11, 2, 5, 3
    q, k, v, g, _ = _inputs(B, T, H, K, V, gate, 5)
    h0 = RNG.standard_normal((B, H, K, V))
    beta = np.zeros((B, T, H))
    o, ht = oracle.forward(q, k, v, g, beta, scale=0.9, h0=h0)
    gk = g if gate == "vector" else np.broadcast_to(g[..., None], (B, T, H, K))
    G = np.cumsum(gk, axis=1)
    for h in range(H):
        for t in range(T):
            St = np.exp(G[0, t, h])[:, None] * h0[0, h]
            np.testing.assert_allclose(o[0, t, h], St.T @ (0.9 * q[0, t, h]), rtol=1e-13,
                                       atol=1e-14)
        np.testing.assert_allclose(ht[0, h], np.exp(G[0, -1, h])[:, None] * h0[0, h],
                                   rtol=1e-13, atol=1e-14)


def test_deltanet_transition_eigenvalues():
    """KDA blog section 2.3: for a unit key the DeltaNet transition
    I - beta k k^T has eigenvalue 1 - beta along k and 1 orthogonal to it."""
    K, V = 6, 4
    k = _unit(RNG.standard_normal(K))
    beta = 0.37
    x = RNG.standard_normal(V)
    u = RNG.standard_normal(K)
    u -= (u @ k) * k
    z = np.zeros((1, 1, 1, V))
    for S0, lam in [(np.outer(k, x), 1 - beta), (np.outer(u, x), 1.0)]:
        _, ht = oracle.forward(np.zeros((1, 1, 1, K)), k.reshape(1, 1, 1, K), z, None,
                               np.full((1, 1, 1), beta), scale=1.0, h0=S0.reshape(1, 1, K, V))
        np.testing.assert_allclose(ht[0, 0], lam * S0, atol=1e-14)


def test_four_token_worked_chunk():
    """KDA blog section 6 (four-token worked chunkwise derivation), written in
    that page's own convention: state [V, K], provisional errors, the
    coefficients rho_ij = beta_i <k_j| D_{j+1:i} |k_i>, chi_ij = s <k_j|D_{j+1:i}|q_i>,
    E_c = Ebar_c (A^kk)^T, S_{c+1} = S_c D_{0:3} + E_c K^end and
    O_c = s S_c Q^boundary + E_c (A^qk)^T."""
    K, V, s = 5, 3, 0.8
    q, k, v, g, beta = _inputs(1, 4, 1, K, V, "vector", 6)
    Sc = RNG.standard_normal((V, K))  # [V, K] state of that page
    al = np.exp(g[0, :, 0])  # retention vectors alpha_i
    Dm = [np.diag(al[i]) for i in range(4)]

    def Dr(a, b):  # D_{a:b} = D_a ... D_b, identity if empty
        out = np.eye(K)
        for i in range(a, b + 1):
            out = out @ Dm[i]
        return out

    kk, qq, vv, bb = k[0, :, 0], q[0, :, 0], v[0, :, 0], beta[0, :, 0]
    ebar = np.stack([bb[i] * (vv[i] - Sc @ Dr(0, i) @ kk[i]) for i in range(4)], axis=1)
    Rc = np.zeros((4, 4))
    Aqk = np.zeros((4, 4))
    for i in range(4):
        for j in range(4):
            if j < i:
                Rc[i, j] = bb[i] * kk[j] @ Dr(j + 1, i) @ kk[i]
            if j <= i:
                Aqk[i, j] = s * kk[j] @ Dr(j + 1, i) @ qq[i]
    Akk = np.linalg.inv(np.eye(4) + Rc)
    Ec = ebar @ Akk.T
    Kend = np.stack([kk[i] @ Dr(i + 1, 3) for i in range(4)], axis=0)
    S_next = Sc @ Dr(0, 3) + Ec @ Kend
    Qb = np.stack([Dr(0, i) @ qq[i] for i in range(4)], axis=1)
    Oc = s * Sc @ Qb + Ec @ Aqk.T
    o, ht = oracle.forward(q, k, v, g, beta, scale=s, h0=Sc.T.reshape(1, 1, K, V))
    np.testing.assert_allclose(o[0, :, 0], Oc.T, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], S_next.T, rtol=1e-12, atol=1e-13)


def test_split_resume_and_varlen():
    """Chunks never change the recurrence: running [0, t1) then [t1, T) with the
    final state handed over equals one run (bitwise, same operation order); a
    packed varlen batch equals independent runs; in reverse mode dh0 of the
    second half is the terminal adjoint of the first."""
    B, T, H, K, V = 1, 40, 2, 6, 5
    q, k, v, g, beta = _inputs(B, T, H, K, V, "vector", 7)
    dO = RNG.standard_normal((B, T, H, V))
    h0 = RNG.standard_normal((1, H, K, V))
    dht = RNG.standard_normal((1, H, K, V))
    o, ht = oracle.forward(q, k, v, g, beta, scale=0.4, h0=h0)
    t1 = 17
    o1, h1 = oracle.forward(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], scale=0.4,
                            h0=h0)
    o2, h2 = oracle.forward(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], scale=0.4,
                            h0=h1)
    assert np.array_equal(np.concatenate([o1, o2], 1), o) and np.array_equal(h2, ht)
    gr = oracle.backward(q, k, v, g, beta, dO, scale=0.4, h0=h0, dht=dht)
    g2 = oracle.backward(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], dO[:, t1:],
                         scale=0.4, h0=h1, dht=dht)
    g1 = oracle.backward(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], dO[:, :t1],
                         scale=0.4, h0=h0, dht=g2["dh0"])
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        np.testing.assert_allclose(np.concatenate([g1[n], g2[n]], 1), gr[n], rtol=1e-12,
                                   atol=1e-13)
    np.testing.assert_allclose(g1["dh0"], gr["dh0"], rtol=1e-12, atol=1e-13)
    # varlen packing
    cu = [0, 5, 5 + 13, 40]
    hv = RNG.standard_normal((3, H, K, V))
    ov, htv = oracle.forward(q, k, v, g, beta, scale=0.4, h0=hv, cu_seqlens=cu)
    gv = oracle.backward(q, k, v, g, beta, dO, scale=0.4, h0=hv, dht=None, cu_seqlens=cu)
    for n in range(3):
        a, e = cu[n], cu[n + 1]
        oi, hi = oracle.forward(q[:, a:e], k[:, a:e], v[:, a:e], g[:, a:e], beta[:, a:e],
                                scale=0.4, h0=hv[n:n + 1])
        gi = oracle.backward(q[:, a:e], k[:, a:e], v[:, a:e], g[:, a:e], beta[:, a:e],
                             dO[:, a:e], scale=0.4, h0=hv[n:n + 1])
        assert np.array_equal(ov[:, a:e], oi) and np.array_equal(htv[n], hi[0])
        for nm in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.array_equal(gv[nm][:, a:e], gi[nm])
        assert np.array_equal(gv["dh0"][n], gi["dh0"][0])


# --------------------------------------------------------------- backward pins

def _loss(args, dO, dht, scale, cu=None, erase=None, write=None):
    q, k, v, g, beta, h0 = args
    o, ht = oracle.forward(q, k, v, g, beta, scale=scale, h0=h0, cu_seqlens=cu, erase=erase,
                           write=write)
    return float((o * dO).sum() + (ht * dht).sum())


@pytest.mark.parametrize("gate,T,K,V,cu", [
    ("none", 1, 4, 4, None), ("vector", 3, 5, 3, None), ("scalar", 63, 4, 6, None),
    ("vector", 64, 3, 4, None), ("vector", 65, 4, 3, None), ("scalar", 130, 3, 3, None),
    ("vector", 70, 16, 24, None), ("vector", 50, 4, 5, [0, 7, 30, 50]),
])
def test_backward_central_differences(gate, T, K, V, cu):
    """Central finite differences of l = <dO, o> + <dht, ht> against the
    hand-derived reverse mode, on every input: a random direction per tensor
    plus random single elements."""
    B = 1 if cu is not None else 2
    H = 2
    q, k, v, g, beta = _inputs(B, T, H, K, V, gate, 100 + T)
    N = B if cu is None else len(cu) - 1
    h0 = RNG.standard_normal((N, H, K, V)) * 0.3
    dO = RNG.standard_normal((B, T, H, V))
    dht = RNG.standard_normal((N, H, K, V))
    if T % 3 == 0:
        beta[..., ::3] = 0.0  # zero beta rows: the undivided beta gradient must hold
    s = K ** -0.5
    gr = oracle.backward(q, k, v, g, beta, dO, scale=s, h0=h0, dht=dht, cu_seqlens=cu)
    args = [q, k, v, g, beta, h0]
    grads = [gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["dbeta"], gr["dh0"]]
    r = np.random.default_rng(T)
    for idx, (x, dx) in enumerate(zip(args, grads)):
        if x is None:
            assert dx is None
            continue
        dirs = [r.standard_normal(x.shape)]
        for _ in range(8):
            e = np.zeros(x.size)
            e[r.integers(x.size)] = 1.0
            dirs.append(e.reshape(x.shape))
        for d in dirs:
            eps = 1e-6 * max(1.0, float(np.abs(x).max()))
            ap = list(args); ap[idx] = x + eps * d
            am = list(args); am[idx] = x - eps * d
            fd = (_loss(ap, dO, dht, s, cu) - _loss(am, dO, dht, s, cu)) / (2 * eps)
            an = float((dx * d).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (idx, fd, an)
    # terminal-state adjoint by linearity: d l / d dht = ht
    _, ht = oracle.forward(q, k, v, g, beta, scale=s, h0=h0, cu_seqlens=cu)
    l1 = _loss(args, dO, dht, s, cu)
    l0 = _loss(args, dO, np.zeros_like(dht), s, cu)
    np.testing.assert_allclose(l1 - l0, (ht * dht).sum(), rtol=1e-12)


def test_separate_erase_write_gradients():
    """Independent erase/write gates (ReWY paper Table 1, GDN2 row) have their
    own gradients; central differences on both."""
    B, T, H, K, V = 1, 20, 1, 4, 3
    q, k, v, g, _ = _inputs(B, T, H, K, V, "vector", 8)
    er = RNG.uniform(0.1, 0.9, size=(B, T, H, K))
    wr = RNG.uniform(0.1, 0.9, size=(B, T, H, V))
    dO = RNG.standard_normal((B, T, H, V))
    dht = RNG.standard_normal((B, H, K, V))
    gr = oracle.backward(q, k, v, g, None, dO, scale=0.5, dht=dht, erase=er, write=wr)
    args = [q, k, v, g, None, None]
    for which, x, dx in (("erase", er, gr["derase"]), ("write", wr, gr["dwrite"])):
        d = RNG.standard_normal(x.shape)
        eps = 1e-6
        kw_p = dict(erase=er, write=wr); kw_p[which] = x + eps * d
        kw_m = dict(erase=er, write=wr); kw_m[which] = x - eps * d
        fd = (_loss(args, dO, dht, 0.5, **kw_p) - _loss(args, dO, dht, 0.5, **kw_m)) / (2 * eps)
        assert abs(fd - (dx * d).sum()) < 1e-6 * max(1, abs(fd))


# ------------------------------------------------------- chunked evaluation pins

@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
@pytest.mark.parametrize("chunk", [4, 16, 64, "nonuniform"])
def test_chunked_matches_token_recurrence(gate, chunk):
    """The chunked WY forward and ReWY backward (ReWY paper Appendix A, Algorithm
    1, Appendix 7 and 10) reach the recurrence's results exactly: agreement to
    ~1e-12 for several chunk sizes, tails, a nonuniform partition (Appendix
    10.1: each chunk length has its own unit-triangular system) and packed
    sequences."""
    B, T, H, K, V = (1, 77, 2, 8, 6)
    q, k, v, g, beta = _inputs(B, T, H, K, V, gate, 9)
    beta[0, 5, 0] = 0.0
    cu = [0, 30, 77] if chunk != "nonuniform" else None
    N = 2 if cu else 1
    h0 = RNG.standard_normal((N, H, K, V)) * 0.2
    dht = RNG.standard_normal((N, H, K, V)) * 0.2
    dO = RNG.standard_normal((B, T, H, V))
    ch = [5, 16, 1, 33, 22] if chunk == "nonuniform" else chunk
    o, ht = oracle.forward(q, k, v, g, beta, scale=0.35, h0=h0, cu_seqlens=cu)
    gr = oracle.backward(q, k, v, g, beta, dO, scale=0.35, h0=h0, dht=dht, cu_seqlens=cu)
    routes = ["rewy", "expanded"] + (["gram_eliminated", "gram_matrix"] if gate == "scalar" else [])
    for route in routes:
        c = chunked.forward_backward(q, k, v, g, beta, dO, scale=0.35, h0=h0, dht=dht,
                                     cu_seqlens=cu, chunk=ch, route=route)
        pairs = [("o", o), ("ht", ht), ("dq", gr["dq"]), ("dk", gr["dk"]), ("dv", gr["dv"]),
                 ("dbeta", gr["dbeta"]), ("dh0", gr["dh0"])]
        if g is not None:
            pairs.append(("dg", gr["dg"]))
        for name, ref in pairs:
            err = np.abs(c[name] - ref).max() / np.abs(ref).max()
            assert err < 1e-12, (route, name, err)


def test_rewy_theorem_matches_expanded_graph():
    """ReWY paper Theorem 3.1 / Appendix 7.1: the shared sensitivity P = A^T Rbar
    equals the expanded graph's Zbar, D = -tril_strict(P R^T) equals its
    two-sided inverse pullback, and E^T P = W^T Rbar (the scan term)."""
    n, K, V = 13, 7, 5
    q, k, v, g, beta = _inputs(1, n, 1, K, V, "vector", 10)
    S = RNG.standard_normal((K, V))
    Sp = RNG.standard_normal((K, V))
    dO = RNG.standard_normal((n, V))
    ctx, res = chunked.chunk_intermediates(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                           beta[0, :, 0], dO, S, Sp, scale=0.3)
    for key in ("P", "D", "Ebar", "Ybar", "dS"):
        np.testing.assert_allclose(res["rewy"][key], res["expanded"][key], rtol=1e-11,
                                   atol=1e-12)
    P = res["rewy"]["P"]
    np.testing.assert_allclose(ctx["E"].T @ P, ctx["W"].T @ res["rewy"]["Rbar"], rtol=1e-11,
                               atol=1e-12)
    # the residual equation itself: M R = Z - E S
    M = np.eye(n) + ctx["L"]
    np.testing.assert_allclose(M @ ctx["R"], ctx["Z"] - ctx["E"] @ S, rtol=1e-12, atol=1e-12)


def test_matrix_intra_centering_invariance():
    """ReWY paper section 3.3 / Appendix 8: replacing gamma, 1/gamma by
    exp(G - c), exp(c - G) for any feature centre c leaves the contraction
    gamma * (H Y) unchanged; with the midpoint centre the factors are bounded by
    exp(Delta / 2)."""
    n, K = 16, 6
    r = np.random.default_rng(11)
    G = np.cumsum(-np.abs(r.standard_normal((n, K))) * 3, axis=0)
    Kt = r.standard_normal((n, K))
    Hm = np.tril(r.standard_normal((n, n)))
    ref = np.exp(G) * (Hm @ (Kt / np.exp(G)))
    for c in (G.max(0), G.min(0), (G.max(0) + G.min(0)) / 2, r.standard_normal(K)):
        alpha, zeta = np.exp(G - c), np.exp(c - G)
        np.testing.assert_allclose(alpha * (Hm @ (Kt * zeta)), ref, rtol=1e-10, atol=1e-12)
    c = (G.max(0) + G.min(0)) / 2
    half = (G.max(0) - G.min(0)) / 2
    assert np.all(np.abs(G - c) <= half + 1e-12)


def test_flop_closed_form_matches_paper():
    """ReWY paper: 7.34M dense FLOPs for the seven-product local WY graph and
    4.19M for ReWY at n = 64, d = 128 (42.9 percent removed)."""
    from chunkwise_delta_rule_chunk_amd import flops
    fx = json.load(open(os.path.join(GOLDEN, "flop_counts.json")))
    n, dk, dv = fx["n"], fx["dk"], fx["dv"]
    ex = flops.local_wy_expanded(n, dk, dv)
    rw = flops.local_wy_rewy(n, dk, dv)
    assert round(ex / 1e6, 2) == fx["expanded_millions_printed"]
    assert round(rw / 1e6, 2) == fx["rewy_millions_printed"]
    assert round(100 * (ex - rw) / ex, 1) == fx["removed_percent_printed"]
    assert ex - rw == 4 * n * n * dk + 4 * n ** 3


def test_kda_gate_formula_and_reverse_mode():
    """GDN2 spec section 4.4: g = -exp(A_log) softplus(x + dt_bias).  At
    x = -dt_bias softplus is ln 2; far on the positive side it is the identity;
    the reverse mode (dx, dA_log, ddt_bias) matches central differences."""
    rng = np.random.default_rng(3)
    B, T, H, K = 2, 5, 3, 4
    x = rng.normal(size=(B, T, H, K))
    a = rng.uniform(-2.0, 0.0, H)
    d = rng.normal(size=(H, K)) * 0.5
    at_zero = oracle.kda_gate(np.broadcast_to(-d, (B, T, H, K)), a, d)
    assert np.allclose(at_zero, -np.exp(a)[None, None, :, None] * np.log(2.0), rtol=1e-14, atol=0)
    far = oracle.kda_gate(np.broadcast_to(40.0 - d, (B, T, H, K)), a, d)
    assert np.allclose(far, -np.exp(a)[None, None, :, None] * 40.0, rtol=1e-12, atol=0)
    R = rng.normal(size=(B, T, H, K))
    dx, da, dd = oracle.kda_gate_backward(x, a, d, R)
    loss = lambda xx, aa, db: float((R * oracle.kda_gate(xx, aa, db)).sum())
    eps = 1e-6
    for grad, arg in ((dx, 0), (da, 1), (dd, 2)):
        base = [x, a, d]
        u = rng.normal(size=base[arg].shape)
        plus, minus = list(base), list(base)
        plus[arg] = base[arg] + eps * u
        minus[arg] = base[arg] - eps * u
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert abs(fd - float((grad * u).sum())) <= 1e-7 * max(1.0, abs(fd)), (arg, fd)


def test_kda_gate_bounded_form_and_reverse_mode():
    """GDN2 spec section 3 (the recurrent kernel's gate) with the bound of
    section 4.3: g = lower_bound * sigmoid(exp(A_log) (x + dt_bias)).  At
    x = -dt_bias it is lower_bound / 2; far on either side it reaches 0 and
    lower_bound; it stays inside (lower_bound, 0); the reverse mode matches
    central differences."""
    rng = np.random.default_rng(5)
    B, T, H, K = 2, 5, 3, 4
    lb = -3.5
    x = rng.normal(size=(B, T, H, K))
    a = rng.uniform(-2.0, 0.0, H)
    d = rng.normal(size=(H, K)) * 0.5
    mid = oracle.kda_gate(np.broadcast_to(-d, (B, T, H, K)), a, d, lb)
    assert np.allclose(mid, lb / 2, rtol=1e-15, atol=0)
    lo = oracle.kda_gate(np.broadcast_to(-2000.0 - d, (B, T, H, K)), a, d, lb)
    hi = oracle.kda_gate(np.broadcast_to(2000.0 - d, (B, T, H, K)), a, d, lb)
    assert np.abs(lo).max() < 1e-20 and np.allclose(hi, lb, rtol=1e-15, atol=0)
    g = oracle.kda_gate(x, a, d, lb)
    assert (g < 0).all() and (g > lb).all()
    # the two forms differ: the bounded one is not the softplus one
    assert not np.allclose(g, oracle.kda_gate(x, a, d))
    R = rng.normal(size=(B, T, H, K))
    dx, da, dd = oracle.kda_gate_backward(x, a, d, R, lb)
    loss = lambda xx, aa, db: float((R * oracle.kda_gate(xx, aa, db, lb)).sum())
    eps = 1e-6
    for grad, arg in ((dx, 0), (da, 1), (dd, 2)):
        base = [x, a, d]
        u = rng.normal(size=base[arg].shape)
        plus, minus = list(base), list(base)
        plus[arg] = base[arg] + eps * u
        minus[arg] = base[arg] - eps * u
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert abs(fd - float((grad * u).sum())) <= 1e-7 * max(1.0, abs(fd)), (arg, fd)


# ------------------------------------------------------ operand-format experiment

def _round_bf16(x):
    """Round to the nearest bfloat16 (ties to even) through the float32 bit
    pattern: keep the top 16 bits after adding half an ulp of the kept part."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_bf16_rounding_helper():
    """bfloat16 keeps 8 significant bits (spacing 2^-7 above 1): 1 + 2^-8 is a
    tie that rounds to 1 (even), 1 + 3 * 2^-8 a tie that rounds up to
    1 + 2^-6, and the relative error of any normal value is at most the unit
    roundoff 2^-8."""
    one = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5])
    r = _round_bf16(one)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2.0 ** -6 and r[3] == -2.5
    x = np.random.default_rng(3).standard_normal(100000) * 10.0 ** np.random.default_rng(4).uniform(-20, 20, 100000)
    rel = np.abs(_round_bf16(x) - x) / np.abs(x)
    assert rel.max() <= 2.0 ** -8 * (1 + 1e-12) and rel.max() > 2.0 ** -8 * 0.9


@pytest.mark.parametrize("strong", [False, True], ids=["kda", "strong_decay"])
def test_precision_of_bf16_D_and_Hq_operands(strong):
    """What bfloat16 operands for the two coefficient matrices D and Hq do to
    the gradients (ReWY paper, "Execution and numerical precision" and the
    precision-eligibility appendix: existing FP32 L/D working matrices keep
    their format there).  The GPU chunk backward forms D and Hq in FP32
    accumulators and feeds them to its products as bfloat16 MFMA operands;
    this measures that rounding alone in the FP64 chunked evaluation at the
    KDA gates (A_log ~ U(-2, 0)) and the strong-decay gates (A_log ~ U(0, 1),
    in-chunk log decay down to about -220), K = V = 128, four chunks.

    Structural pins: dv and dh0 do not depend on D or Hq, so they are
    unchanged bit for bit.  Measured: dq 1.7e-3, dk 1.4e-3, dg 1.3e-3,
    dbeta 8e-5 relative (normwise) in both regimes -- below the bfloat16
    unit roundoff 2^-8 and below the 3.5e-3 the whole bfloat16 GPU path
    shows on dv, which involves neither matrix."""
    import workloads

    inp = workloads.make_inputs(1, 256, 2, 128, 128, gate="vector", dtype="bf16", seed=7,
                                strong=strong, dht=True)
    f64 = lambda t: None if t is None else t.double().numpy()
    args = [f64(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.dO)]
    kw = dict(scale=inp.scale, h0=f64(inp.h0), dht=f64(inp.dht))
    exact = chunked.forward_backward(*args, **kw)
    rounded = chunked.forward_backward(*args, **kw, round_DH=_round_bf16)
    err = {n: np.linalg.norm(rounded[n] - exact[n]) / np.linalg.norm(exact[n])
           for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0")}
    assert err["dv"] == 0.0 and err["dh0"] == 0.0, err
    for n in ("dq", "dk", "dg"):
        assert 5e-4 < err[n] < 2.5e-3, (n, err)
    assert err["dbeta"] < 2e-4, err
    # the gates of the strong regime really are strong: some in-chunk log
    # decay falls below -100 there, none does at the KDA gates
    g = args[3][0]
    low = min(np.cumsum(g[c:c + 64], axis=0).min() for c in range(0, 256, 64))
    assert (low < -100.0) == strong, low
