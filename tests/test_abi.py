"""C-ABI checks that need no GPU: the library loads, exports every function
include/rewy.h declares, and rejects malformed descriptors on the host before
anything is enqueued."""
import ctypes
import os
import re

import pytest

from chunkwise_delta_rule_chunk_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "rewy.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rewy_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("librewy.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_symbol(lib):
    decl = _declared()
    assert decl == sorted(B.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\bT (rewy_[a-z0-9_]+)\b", out)))
    assert exported == decl  # nothing else of ours is exported


def _desc(**kw):
    d = dict(B=1, T=256, H=2, K=128, V=128, N=0, cu_seqlens=None, cu_seqlens_host=None,
             dtype=B.REWY_BF16, beta_dtype=B.REWY_BF16, gate=B.REWY_GATE_VECTOR,
             policy=B.REWY_RECOMPUTE, scale=128 ** -0.5)
    d.update(kw)
    return B.RewyDesc(**d)


def test_status_strings(lib):
    assert B.rewy_status_string(0) == "REWY_OK"
    assert B.rewy_status_string(-1) == "REWY_EINVAL"
    assert B.rewy_status_string(-2) == "REWY_EUNSUPPORTED"
    assert B.rewy_status_string(-3) == "REWY_EWORKSPACE"
    assert B.rewy_status_string(-4) == "REWY_EHIP"
    assert B.rewy_status_string(99) == "REWY_UNKNOWN"


@pytest.mark.parametrize("bad,msg", [
    (dict(K=48), "not supported"), (dict(V=256), "not supported"), (dict(K=300), "exceeds 256"),
    (dict(B=0), "bad shape"), (dict(H=-1), "bad shape"), (dict(dtype=7), "bad dtype"),
    (dict(gate=3), "bad gate"), (dict(policy=5), "bad policy"),
    (dict(dtype=B.REWY_F32, K=128), "not supported"), (dict(N=3), "must equal B"),
])
def test_invalid_descriptor_rejected(lib, bad, msg):
    assert B.rewy_workspace_bytes(_desc(**bad), 0) == 0
    assert msg in B.rewy_last_error()


def test_cu_seqlens_validation(lib):
    cu = (ctypes.c_int32 * 4)(0, 10, 5, 256)  # not ascending
    d = _desc(N=3, cu_seqlens=8, cu_seqlens_host=ctypes.addressof(cu))
    assert B.rewy_workspace_bytes(d, 0) == 0 and "not ascending" in B.rewy_last_error()
    cu2 = (ctypes.c_int32 * 3)(0, 100, 200)  # does not end at T
    d = _desc(N=2, cu_seqlens=8, cu_seqlens_host=ctypes.addressof(cu2))
    assert B.rewy_workspace_bytes(d, 0) == 0 and "end at T" in B.rewy_last_error()
    d = _desc(B=2, N=2, cu_seqlens=8)
    assert B.rewy_workspace_bytes(d, 0) == 0 and "B == 1" in B.rewy_last_error()


def test_layout_does_not_depend_on_the_host_copy_of_cu_seqlens(lib):
    """Workspace and saved sizes (and so every buffer offset) are the same
    with and without the optional host copy of cu_seqlens, so a caller may pass
    it to one call and not to another; the layout is sized by the bound
    ceil(T / 64) + N chunk slots."""
    cu = (ctypes.c_int32 * 4)(0, 5, 69, 256)
    for policy in (B.REWY_RECOMPUTE, B.REWY_SAVE):
        with_host = _desc(N=3, cu_seqlens=8, cu_seqlens_host=ctypes.addressof(cu), policy=policy)
        without = _desc(N=3, cu_seqlens=8, policy=policy)
        for phase in (0, 1, 2):
            assert B.rewy_workspace_bytes(with_host, phase) == B.rewy_workspace_bytes(without, phase) > 0
        assert B.rewy_saved_bytes(with_host) == B.rewy_saved_bytes(without)
    # sized by the bound: 256 / 64 + 3 = 7 chunk slots, as many as an unpacked
    # 448-token sequence has (every buffer is sized by the chunk slots)
    for phase in (0, 1):
        assert B.rewy_workspace_bytes(_desc(N=3, cu_seqlens=8), phase) == \
            B.rewy_workspace_bytes(_desc(T=7 * 64), phase)


def test_workspace_sizes_follow_the_layout(lib):
    d = _desc()
    nc = 4  # 256 tokens / 64
    e, H, K, V, BT = 2, 2, 128, 128, 256
    up = lambda x: (x + 255) // 256 * 256
    tokK, tokV = up(BT * H * K * e), up(BT * H * V * e)
    tileK, tile64 = up(nc * H * K * 64 * e), up(nc * H * 64 * 64 * e)
    head = up(nc * 16) + up(2 * 4) + up(1 * 4)  # chunk records, seqoff [N+1], scan order [N]
    tileV = up(nc * H * V * 64 * e)
    glast = up(nc * H * K * 4)
    states = up(nc * H * K * V * e) + tileV                             # hbuf, R
    scan = tokK + tileK + tokV                                          # W, Ft, U
    out = tileK + tile64                                                # Qg, Cq
    rscan = tokK + 2 * tileK + tile64                                   # F, Wt, Qgt, Cqt
    rscan += tile64                                                     # At (no G2 tile: vector gate)
    rscan += up(nc * H * 4 * K * 16)                                    # Gst
    bwd = up(nc * H * V * 64 * e) + up(nc * H * K * V * e)              # Rbt, dhbuf
    shared = glast + states
    # the forward of the recompute policy needs no per-chunk states or corrections
    assert B.rewy_workspace_bytes(d, 0) == head + glast + scan + out
    # the backward's buffers reuse the output operands' space
    assert B.rewy_workspace_bytes(d, 1) == head + glast + scan + states + rscan + bwd
    # the gate formed in the kernels: per (chunk, head, wave) partial sums of
    # ddt_bias [K] and dA_log [1] follow the backward's buffers
    assert B.rewy_workspace_bytes(d, 2) == head + glast + scan + states + rscan + bwd + up(nc * H * 4 * (K + 1) * 4)
    assert B.rewy_workspace_bytes(_desc(gate=B.REWY_GATE_SCALAR), 2) == 0
    assert "VECTOR" in B.rewy_last_error()
    assert B.rewy_workspace_bytes(d, 3) == 0 and "bad phase" in B.rewy_last_error()
    assert B.rewy_saved_bytes(d) == 0
    ds = _desc(policy=B.REWY_SAVE)
    assert B.rewy_saved_bytes(ds) == shared + rscan
    assert B.rewy_workspace_bytes(ds, 0) == head + scan + out
    assert B.rewy_workspace_bytes(ds, 1) == head + bwd


def test_calls_reject_bad_pointers_without_launching(lib):
    d = _desc()
    ws = ctypes.create_string_buffer(1024)
    P = ctypes.c_void_p
    # q is NULL: host-side rejection, nothing enqueued
    rc = B.rewy_fwd(d, None, P(256), P(256), P(256), P(256), None, P(256), None, None,
                    P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "q is NULL" in B.rewy_last_error()
    # missing gate for a gated descriptor
    rc = B.rewy_fwd(d, P(256), P(256), P(256), None, P(256), None, P(256), None, None,
                    P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "g must be given" in B.rewy_last_error()
    # workspace too small
    rc = B.rewy_fwd(d, P(256), P(256), P(256), P(256), P(256), None, P(256), None, None,
                    P(256), 16, None)
    assert rc == B.REWY_EWORKSPACE
    # misaligned tensor
    rc = B.rewy_fwd(d, P(258), P(256), P(256), P(256), P(256), None, P(256), None, None,
                    P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "aligned" in B.rewy_last_error()
    # h0 without dh0 in the backward
    rc = B.rewy_bwd(d, P(256), P(256), P(256), P(256), P(256), P(256), P(256), None, None,
                    P(256), P(256), P(256), P(256), P(256), None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "dh0" in B.rewy_last_error()
    # dg missing for a gated backward
    rc = B.rewy_bwd(d, P(256), P(256), P(256), P(256), P(256), None, P(256), None, None,
                    P(256), P(256), P(256), None, P(256), None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "dg" in B.rewy_last_error()
    # save-all policy without the saved buffer
    dsv = _desc(policy=B.REWY_SAVE)
    rc = B.rewy_fwd(dsv, P(256), P(256), P(256), P(256), P(256), None, P(256), None, None,
                    P(256), 1 << 40, None)
    assert rc == B.REWY_EWORKSPACE
    # token-serial forward: the same host-side checks
    rc = B.rewy_recurrent_fwd(d, None, P(256), P(256), P(256), P(256), None, P(256), None, None)
    assert rc == B.REWY_EINVAL and "q is NULL" in B.rewy_last_error()
    rc = B.rewy_recurrent_fwd(d, P(256), P(256), P(256), None, P(256), None, P(256), None, None)
    assert rc == B.REWY_EINVAL and "g must be given" in B.rewy_last_error()
    rc = B.rewy_recurrent_fwd(d, P(256), P(256), P(264), P(256), P(256), None, P(256), None, None)
    assert rc == B.REWY_EINVAL and "aligned" in B.rewy_last_error()
    rc = B.rewy_recurrent_fwd_gdn2(d, P(256), P(256), P(256), P(256), None, P(256), None, P(256),
                                   None, None)
    assert rc == B.REWY_EINVAL and "b and w" in B.rewy_last_error()
    rc = B.rewy_recurrent_fwd_gdn2(_desc(beta_dtype=B.REWY_F32), P(256), P(256), P(256), P(256),
                                   P(256), P(256), None, P(256), None, None)
    assert rc == B.REWY_EUNSUPPORTED
    # gate formed in the kernels: vector gate only, every gate tensor given, aligned
    rc = B.rewy_fwd_kda_gate(_desc(gate=B.REWY_GATE_SCALAR), P(256), P(256), P(256), P(256), P(256),
                             P(256), 0.0, P(256), None, P(256), None, None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "VECTOR" in B.rewy_last_error()
    rc = B.rewy_fwd_kda_gate(d, P(256), P(256), P(256), P(256), None, P(256), 0.0, P(256), None, P(256),
                             None, None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "A_log" in B.rewy_last_error()
    rc = B.rewy_fwd_kda_gate(d, P(256), P(256), P(256), P(256), P(256), P(264), 0.0, P(256), None, P(256),
                             None, None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "aligned" in B.rewy_last_error()
    # the bounded form's lower bound lies in [-5, 0); 0 selects the softplus form
    for lb in (-5.5, 0.5, float("nan")):
        rc = B.rewy_fwd_kda_gate(d, P(256), P(256), P(256), P(256), P(256), P(256), lb, P(256), None,
                                 P(256), None, None, P(256), 1 << 40, None)
        assert rc == B.REWY_EINVAL and "lower_bound" in B.rewy_last_error(), lb
    rc = B.rewy_bwd_kda_gate(d, P(256), P(256), P(256), P(256), P(256), P(256), 0.0, P(256), None,
                             P(256), None, None, P(256), P(256), P(256), P(256), None, P(256), P(256),
                             None, P(256), 1 << 40, None)
    assert rc == B.REWY_EINVAL and "dA_log" in B.rewy_last_error()
    # the phase-1 size is too small for the backward with the gate in the kernels
    n1 = B.rewy_workspace_bytes(d, 1)
    rc = B.rewy_bwd_kda_gate(d, P(256), P(256), P(256), P(256), P(256), P(256), -1.0, P(256), None,
                             P(256), None, None, P(256), P(256), P(256), P(256), P(256), P(256),
                             P(256), None, P(256), n1, None)
    assert rc == B.REWY_EWORKSPACE
    del ws


def test_noalloc_forward_rejects_problems_beyond_its_scratch(lib):
    """rewy_fwd_noalloc refuses, on the host and before touching any device, a
    problem whose forward workspace exceeds the fixed device scratch."""
    P = ctypes.c_void_p
    big = _desc(B=1, T=65536, H=32)  # about 4.7 GB of workspace
    assert B.rewy_workspace_bytes(big, 0) > B.NOALLOC_SCRATCH_BYTES
    rc = B.rewy_fwd_noalloc(big, P(256), P(256), P(256), P(256), P(256), None, P(256), None, None,
                            None)
    assert rc == B.REWY_EWORKSPACE
    assert "rewy_fwd_noalloc" in B.rewy_last_error() and "scratch" in B.rewy_last_error()
    # argument errors come first, as for rewy_fwd
    rc = B.rewy_fwd_noalloc(_desc(K=48), P(256), P(256), P(256), P(256), P(256), None, P(256),
                            None, None, None)
    assert rc == B.REWY_EUNSUPPORTED


def test_backward_schedule_knob(lib):
    """rewy_bwd_schedule sets the chunk backward's schedule; the separate one
    needs a larger backward workspace (P, D and the write part of dbeta handed
    from the producer to the consumers) and no other buffer changes."""
    d = _desc()
    joint = B.rewy_workspace_bytes(d, 1)
    fwd = B.rewy_workspace_bytes(d, 0)
    prev = B.rewy_bwd_schedule(B.REWY_SCHEDULE_SEPARATE)
    try:
        assert prev == B.REWY_SCHEDULE_JOINT
        assert B.rewy_bwd_schedule(-1) == B.REWY_SCHEDULE_SEPARATE
        nc, H, K, V, e = 4, 2, 128, 128, 2
        up = lambda x: (x + 255) // 256 * 256
        extra = up(nc * H * 64 * V * e) + up(nc * H * 4 * 4 * 2 * 64 * 4 * e) \
            + up(nc * H * 4 * 16 * 16 * 4) + up(nc * H * 64 * 4)
        assert B.rewy_workspace_bytes(d, 1) == joint + extra
        assert B.rewy_workspace_bytes(d, 0) == fwd
        with pytest.raises(B.RewyError):
            B.rewy_bwd_schedule(7)
        assert B.rewy_bwd_schedule(-1) == B.REWY_SCHEDULE_SEPARATE
    finally:
        B.rewy_bwd_schedule(prev)
    assert B.rewy_workspace_bytes(d, 1) == joint


def test_product_path_has_no_fallback():
    """The package never imports the oracle and raises when the library is missing."""
    import chunkwise_delta_rule_chunk_amd as pkg
    pkg_dir = os.path.dirname(pkg.__file__)
    for name in os.listdir(pkg_dir):
        if name.endswith(".py"):
            src = open(os.path.join(pkg_dir, name)).read()
            assert "import oracle" not in src and "from oracle" not in src, name
    saved, B._lib, path = B._lib, None, B.LIB_PATH
    try:
        B.LIB_PATH = path + ".missing"
        with pytest.raises(RuntimeError, match="missing"):
            B.load()
    finally:
        B.LIB_PATH, B._lib = path, saved
