"""The C ABI library on the CPU: it loads, exports every function include/pyr.h
declares, and its host-only helpers and argument validation behave as the
header states.  No call here enqueues device work: every call either is a
geometry helper or fails validation, which happens before any HIP call."""

import ctypes
import os

import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import _binding as B
from oracle import reference

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libpyr.so not built (run __graft_entry__.build())")


def _p(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, q_len=4096, kv_len=4096,
                branching=4, top_k=8, dtype=torch.bfloat16)
    base.update(kw)
    return H.Problem(**base)


def test_exports_every_declared_function():
    lib = H.lib()
    names = H.declared_functions()
    assert {"pyr_build_pyramid", "pyr_select_topk", "pyr_block_sparse_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert H.pyr_abi_version() == 5


def test_single_hip_runtime_in_process():
    H.lib()
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs


@pytest.mark.parametrize("kv_len,b", [(131072, 4), (32768, 4), (2048, 2), (1048576, 4),
                                      (64 * 37 + 13, 3), (1, 2), (64, 4), (65, 4)])
def test_geometry_matches_oracle(kv_len, b):
    p = _p(q_len=kv_len, kv_len=kv_len, branching=b)
    sizes = reference.level_sizes(reference.num_blocks(kv_len, 64), b)
    assert H.pyr_num_levels(p) == len(sizes)
    assert H.pyr_pyramid_nodes(p) == sum(sizes)
    offs = [sum(sizes[:i]) for i in range(len(sizes))]
    assert [H.pyr_level_offset(p, i) for i in range(len(sizes))] == offs
    assert H.pyr_level_offset(p, len(sizes)) == -1
    assert H.pyr_num_query_blocks(p) == reference.num_blocks(kv_len, 64)
    assert H.pyr_attn_workspace_bytes(p) == 0


def test_pyramid_planes_and_buffer_shape():
    """bf16 problems carry the fp32 plane plus the bf16 hi/lo plane, fp32
    problems only the fp32 plane; the allocation helper sizes the buffer from
    the library's own answer."""
    pb = _p()
    pf = _p(dtype=torch.float32)
    assert H.pyr_pyramid_planes(pb) == 2
    assert H.pyr_pyramid_planes(pf) == 1
    nodes = H.pyr_pyramid_nodes(pb)
    assert H.pyramid_shape(pb) == (pb.batch, pb.n_kv_heads, 2, nodes, pb.head_dim)
    assert H.pyramid_shape(pf) == (pb.batch, pb.n_kv_heads, 1, nodes, pb.head_dim)
    t = H.alloc_pyramid(pb, device="cpu")
    assert tuple(t.shape) == H.pyramid_shape(pb) and t.dtype == torch.float32


def test_decode_geometry():
    p = _p(batch=64, n_q_heads=32, n_kv_heads=8, q_len=1, kv_len=262144, top_k=64)
    assert H.pyr_num_query_blocks(p) == 1
    assert H.pyr_num_levels(p) == 7
    assert H.pyr_pyramid_nodes(p) == 5461
    assert H.pyr_attn_workspace_bytes(p) > 0


@pytest.mark.parametrize("kv_len,hq,hk,d,k", [(1048576, 8, 1, 128, 64), (4096 + 13, 16, 2, 64, 31),
                                              (64, 8, 2, 128, 63), (8192, 128, 8, 128, 15),
                                              (131072, 32, 8, 128, 63)])
def test_prefill_transposed_v_workspace(kv_len, hq, hk, d, k):
    """Dense bfloat16 prefill with G = q_heads/kv_heads a multiple of 4 and
    (top_k + 1) * G/4 >= 16 may use a block-transposed copy of v: one
    64 x head_dim bf16 tile per key block of every (batch, KV head).  Other
    prefill problems use no workspace."""
    b = 2
    base = dict(batch=b, n_q_heads=hq, n_kv_heads=hk, head_dim=d, q_len=kv_len, kv_len=kv_len,
                top_k=k)
    nb = reference.num_blocks(kv_len, 64)
    assert H.pyr_attn_workspace_bytes(_p(**base)) == b * hk * nb * 64 * d * 2
    g = hq // hk
    for kw in (dict(n_q_heads=2 * hk), dict(n_q_heads=3 * hk), dict(n_q_heads=hk),
               dict(top_k=(16 * 4) // g - 2),      # just short of the threshold
               dict(dtype=torch.float32), dict(batch=0), dict(q_len=0, kv_len=0)):
        assert H.pyr_attn_workspace_bytes(_p(**dict(base, **kw))) == 0, kw


def _status(fn, *args):
    lib = H.lib()
    return getattr(lib, fn)(*args), lib.pyr_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 3), (dict(n_q_heads=6, n_kv_heads=4), 2), (dict(branching=1), 2),
    (dict(top_k=0), 2), (dict(q_len=100, kv_len=4096), 3), (dict(batch=-1), 2),
    (dict(top_k=2000), 3),
])
def test_invalid_problems_rejected_before_launch(kw, status):
    p = _p(**kw)
    dummy = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    s, msg = _status("pyr_build_pyramid", ctypes.byref(p.c()), dummy, dummy, None)
    assert s == status and msg
    assert H.pyr_num_levels(p) == -1


def test_bad_block_and_dtype():
    p = _p()
    c = p.c()
    c.block = 32
    s, _ = _status("pyr_build_pyramid", ctypes.byref(c), ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert s == 3
    c = p.c()
    c.dtype = 7
    s, _ = _status("pyr_select_topk", ctypes.byref(c), *([ctypes.c_void_p(16)] * 3), None, None, None)
    assert s == 2


def test_null_and_misaligned_pointers():
    p = _p()
    c = ctypes.byref(p.c())
    s, msg = _status("pyr_build_pyramid", c, None, ctypes.c_void_p(16), None)
    assert s == 1 and "NULL" in msg
    s, _ = _status("pyr_build_pyramid", c, ctypes.c_void_p(18), ctypes.c_void_p(16), None)
    assert s == 4
    s, _ = _status("pyr_select_topk", c, ctypes.c_void_p(16), None, ctypes.c_void_p(16), None, None, None)
    assert s == 1
    s, _ = _status("pyr_block_sparse_attn", c, *([ctypes.c_void_p(16)] * 4), None, None, None, 0, None)
    assert s == 1


def test_decode_workspace_required():
    p = _p(q_len=1, kv_len=8192)
    c = ctypes.byref(p.c())
    ptr = ctypes.c_void_p(16)
    s, msg = _status("pyr_block_sparse_attn", c, ptr, ptr, ptr, ptr, ptr, None, None, 0, None)
    assert s == 5 and "workspace" in msg
    need = H.pyr_attn_workspace_bytes(p)
    s, _ = _status("pyr_block_sparse_attn", c, ptr, ptr, ptr, ptr, ptr, None, ptr, need - 1, None)
    assert s == 5


def test_empty_problems_are_noops():
    for kw in (dict(batch=0), dict(q_len=0, kv_len=0)):
        p = _p(**kw)
        c = ctypes.byref(p.c())
        assert _status("pyr_build_pyramid", c, None, None, None)[0] == 0
        assert _status("pyr_select_topk", c, None, None, None, None, None, None)[0] == 0
        assert _status("pyr_block_sparse_attn", c, None, None, None, None, None, None, None, 0,
                       None)[0] == 0


def test_status_strings():
    lib = H.lib()
    for s in range(7):
        assert lib.pyr_status_string(s)


def test_binding_rejects_wrong_shapes_on_host():
    p = _p(q_len=128, kv_len=128)
    k = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        H.pyr_build_pyramid(p, k, torch.zeros(1))


def _bwd(p, ptrs, ws=None, nbytes=0):
    """Call pyr_block_sparse_attn_bwd with the ten tensor pointers `ptrs`
    (q, k, v, sel, o, lse, dout, dq, dk, dv)."""
    return _status("pyr_block_sparse_attn_bwd", ctypes.byref(p.c()), *ptrs, ws, nbytes, None)


def test_backward_validation_before_launch():
    ptr = ctypes.c_void_p(16)
    full = [ptr] * 10
    p = _p()
    need = H.pyr_attn_bwd_workspace_bytes(p)
    nqb, nb = 4096 // 64, 4096 // 64
    # at least the records of 512 bytes per (batch, query head, query block) and
    # the route bitmap; at most that plus metadata and a partial slot per entry
    base = 1 * 4 * nqb * 512 + 1 * 2 * nb * ((nqb + 31) // 32) * 4
    assert base < need <= base + 2 * 1 * 2 * nqb * 9 * (64 * 128 * 8 + 64) + 8192
    s, msg = _bwd(p, full)
    assert s == 5 and "workspace" in msg
    s, _ = _bwd(p, full, ptr, need - 1)
    assert s == 5
    s, _ = _bwd(p, full, ctypes.c_void_p(24), need)
    assert s == 4
    for i in range(10):      # each tensor is required
        ptrs = list(full)
        ptrs[i] = None
        s, msg = _bwd(p, ptrs, ptr, need)
        assert s == 1 and "NULL" in msg
        ptrs[i] = ctypes.c_void_p(18)
        s, _ = _bwd(p, ptrs, ptr, need)
        assert s == 4
    # bfloat16 prefill only
    s, msg = _bwd(_p(dtype=torch.float32), full, ptr, need)
    assert s == 3 and "bfloat16" in msg
    s, msg = _bwd(_p(q_len=1, kv_len=4096), full, ptr, need)
    assert s == 3 and "prefill" in msg
    assert H.pyr_attn_bwd_workspace_bytes(_p(head_dim=96)) == 0


def test_backward_empty_problems_are_noops():
    for kw in (dict(batch=0), dict(q_len=0, kv_len=0)):
        assert _bwd(_p(**kw), [None] * 10)[0] == 0


def test_backward_binding_rejects_wrong_shapes_on_host(monkeypatch):
    # host tensors stand in for device ones so that the shape checks are reached
    orig = B._expect
    monkeypatch.setattr(B, "_expect", lambda t, n, s, d, device_type="cuda": orig(t, n, s, d, "cpu"))
    p = _p(q_len=128, kv_len=128)
    q = torch.zeros((1, 4, 128, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 128, 128), dtype=torch.bfloat16)
    sel = torch.zeros((1, 2, 2, 9), dtype=torch.int32)
    lse = torch.zeros((1, 4, 128))
    with pytest.raises(ValueError, match="dk: shape"):
        H.pyr_block_sparse_attn_bwd(p, q, k, k, sel, q, lse, q, q, q, k, None)
    with pytest.raises(ValueError, match="lse: dtype"):
        H.pyr_block_sparse_attn_bwd(p, q, k, k, sel, q, lse.double(), q, q, k, k, None)
    with pytest.raises(ValueError, match="sel: shape"):
        H.pyr_block_sparse_attn_bwd(p, q, k, k, sel[..., :4], q, lse, q, q, k, k, None)


def test_capacity_geometry():
    """With kv_capacity the layout (levels, offsets, nodes) follows the capacity."""
    p = _p(q_len=1, kv_len=64 * 5 + 3, kv_capacity=64 * 40)
    cap = reference.level_sizes(40, 4)                     # 40/10/3/1
    assert H.pyr_num_levels(p) == len(cap)
    assert H.pyr_pyramid_nodes(p) == sum(cap)
    assert [H.pyr_level_offset(p, l) for l in range(len(cap))] == [sum(cap[:l]) for l in range(len(cap))]
    assert H.pyramid_shape(p)[3] == sum(cap)
    s, msg = _status("pyr_build_pyramid", ctypes.byref(_p(kv_capacity=100).c()), ctypes.c_void_p(16),
                     ctypes.c_void_p(16), None)
    assert s == 2 and "kv_capacity" in msg


def test_append_validation():
    ptr = ctypes.c_void_p(16)
    p = _p(q_len=1, kv_len=1000, kv_capacity=4096)
    c = ctypes.byref(p.c())
    for old in (0, -1, 1001):
        s, msg = _status("pyr_append_pyramid", c, ptr, old, ptr, None)
        assert s == 2 and "old_len" in msg
    assert _status("pyr_append_pyramid", c, None, 1000, None, None)[0] == 0   # nothing to do
    s, _ = _status("pyr_append_pyramid", c, None, 999, ptr, None)
    assert s == 1
    s, _ = _status("pyr_append_pyramid", c, ptr, 999, ctypes.c_void_p(20), None)
    assert s == 4
    # without a capacity the layout follows the length: an append across a
    # block boundary would move every level above the finest
    p0 = _p(q_len=1, kv_len=1000)
    c0 = ctypes.byref(p0.c())
    for old in (900, 960, 1):
        s, msg = _status("pyr_append_pyramid", c0, ptr, old, ptr, None)
        assert s == 2 and "kv_capacity" in msg, (old, msg)
    # within the last block the layout is unchanged: validation goes on (and
    # stops at the missing pointer before anything is launched)
    assert _status("pyr_append_pyramid", c0, None, 961, ptr, None)[0] == 1


def test_backward_rejects_capacity():
    ptr = ctypes.c_void_p(16)
    p = _p(kv_capacity=8192)
    s, msg = _bwd(p, [ptr] * 10, ptr, 1 << 40)
    assert s == 3 and "capacity" in msg


def _packed_c(total=1000, **kw):
    """The C problem of a packed batch of 3 sequences; cu is a stand-in device
    address (validation never dereferences it)."""
    kw = dict(dict(batch=3, q_len=512, kv_len=512), **kw)
    c = _p(**kw).c()
    c.cu = 64
    c.total_len = total
    return c


def test_packed_geometry():
    """A packed problem has the layout of a dense one of length kv_len (the
    bound on every sequence's length)."""
    c = _packed_c()
    dense = _p(batch=3, q_len=512, kv_len=512)
    lib = H.lib()
    assert lib.pyr_num_levels(ctypes.byref(c)) == H.pyr_num_levels(dense)
    assert lib.pyr_pyramid_nodes(ctypes.byref(c)) == H.pyr_pyramid_nodes(dense)
    assert lib.pyr_num_query_blocks(ctypes.byref(c)) == 8
    assert lib.pyr_attn_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.pyr_attn_bwd_workspace_bytes(ctypes.byref(c)) == 0
    g4 = _packed_c(n_q_heads=8)            # packed batches read v directly
    assert lib.pyr_attn_workspace_bytes(ctypes.byref(g4)) == 0


def test_packed_validation():
    ptr = ctypes.c_void_p(16)
    cases = [
        (_packed_c(q_len=1, kv_len=512), 3, "q_len == kv_len"),
        (_packed_c(kv_capacity=1024), 3, "kv_capacity"),
        (_packed_c(total=-1), 2, "total_len"),
    ]
    c = _packed_c()
    c.cu = 66
    cases.append((c, 4, "cu"))
    c = _p().c()
    c.total_len = 10
    cases.append((c, 2, "total_len"))
    for c, status, word in cases:
        s, msg = _status("pyr_build_pyramid", ctypes.byref(c), ptr, ptr, None)
        assert s == status and word in msg, (s, msg)
    c = _packed_c()
    s, msg = _status("pyr_append_pyramid", ctypes.byref(c), ptr, 10, ptr, None)
    assert s == 3 and "packed" in msg
    s, msg = _status("pyr_block_sparse_attn_bwd", ctypes.byref(c), *([ptr] * 10), ptr, 1 << 40, None)
    assert s == 3 and "packed" in msg


def test_packed_empty_is_noop():
    c = ctypes.byref(_packed_c(total=0))
    assert _status("pyr_build_pyramid", c, None, None, None)[0] == 0
    assert _status("pyr_select_topk", c, None, None, None, None, None, None)[0] == 0
    assert _status("pyr_block_sparse_attn", c, None, None, None, None, None, None, None, 0,
                   None)[0] == 0


def test_packed_binding_shapes(monkeypatch):
    """The binding expects [H, total, d] tensors, [H, total] lse and batch+1
    offsets for a packed problem, and checks them before calling the library."""
    orig = B._expect
    monkeypatch.setattr(B, "_expect", lambda t, n, s, d, device_type="cuda": orig(t, n, s, d, "cpu"))
    cu = torch.tensor([0, 100, 300], dtype=torch.int32)
    q = torch.zeros((4, 300, 128), dtype=torch.bfloat16)
    k = torch.zeros((2, 300, 128), dtype=torch.bfloat16)
    p = H.problem_for_packed(q, k, cu, 256, 4, 8)
    assert (p.batch, p.total_len, p.q_len, p.kv_len) == (2, 300, 256, 256)
    assert p.q_shape == (4, 300, 128) and p.kv_shape == (2, 300, 128) and p.lse_shape == (4, 300)
    with pytest.raises(ValueError, match="k: shape"):
        H.pyr_build_pyramid(p, k[:, :200], torch.zeros(H.pyramid_shape(p)))
    with pytest.raises(ValueError, match="cu: shape"):
        H.pyr_build_pyramid(H.Problem(**{**p.__dict__, "cu": cu[:2]}), k,
                            torch.zeros(H.pyramid_shape(p)))
    with pytest.raises(ValueError, match="cu: dtype"):
        H.pyr_build_pyramid(H.Problem(**{**p.__dict__, "cu": cu.long()}), k,
                            torch.zeros(H.pyramid_shape(p)))
    sel = torch.zeros((2, 2, 4, 9), dtype=torch.int32)
    with pytest.raises(ValueError, match="lse: shape"):
        H.pyr_block_sparse_attn(p, q, k, k, sel, q, torch.zeros((4, 2, 150)))


def test_select_budgets_validation():
    p = _p()
    c = ctypes.byref(p.c())
    ptr = ctypes.c_void_p(16)
    for fb_k, margin, kh, status, word in [(9, 0.0, None, 2, "fallback_k"), (-1, 0.0, None, 2, "fallback_k"),
                                           (4, float("nan"), None, 2, "margin"),
                                           (4, float("inf"), None, 2, "margin"),
                                           (4, 0.5, ctypes.c_void_p(18), 4, "k_head")]:
        s, msg = _status("pyr_select_topk_budgets", c, ptr, ptr, kh, fb_k, margin, ptr, None, None,
                         None)
        assert s == status and word in msg, (s, msg)
    e = ctypes.byref(_p(batch=0).c())
    assert _status("pyr_select_topk_budgets", e, None, None, None, 0, 0.0, None, None, None,
                   None)[0] == 0


def test_budgets_from_entropy_matches_the_oracle():
    import numpy as np
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(1, 17))
        ent = rng.random(n).astype(np.float32) * float(rng.choice([0.0, 1.0, 8.0]))
        total = int(rng.integers(0, 300))
        kmin = int(rng.integers(1, 8))
        kmax = kmin + int(rng.integers(0, 64))
        got = H.pyr_budgets_from_entropy([float(x) for x in ent], total, kmin, kmax)
        assert got == reference.budgets_from_entropy([float(x) for x in ent], total, kmin, kmax)
    lib = H.lib()
    out = (ctypes.c_int32 * 2)()
    ent = (ctypes.c_float * 2)(1.0, -1.0)
    assert lib.pyr_budgets_from_entropy(ent, 2, 8, 1, 4, out) == 2
    ent = (ctypes.c_float * 2)(1.0, 1.0)
    assert lib.pyr_budgets_from_entropy(ent, 2, 8, 0, 4, out) == 2
    assert lib.pyr_budgets_from_entropy(ent, 2, 8, 3, 2, out) == 2
    assert lib.pyr_budgets_from_entropy(None, 2, 8, 1, 4, out) == 1
    assert lib.pyr_budgets_from_entropy(None, 0, 8, 1, 4, None) == 0


def _sa(p, ptrs, ws=None, nbytes=0):
    """Call pyr_select_attn with the ten tensor pointers `ptrs` (q, k, v,
    pyramid, sel, trace_ids, trace_scores, o, lse) and a workspace."""
    return _status("pyr_select_attn", ctypes.byref(p.c()), *ptrs, ws, nbytes, None)


def test_select_attn_validation_before_launch():
    ptr = ctypes.c_void_p(16)
    p = _p()
    full = [ptr, ptr, ptr, ptr, ptr, None, None, ptr, None]
    for i in (0, 1, 2, 3, 4, 7):           # q, k, v, pyramid, sel, o may not be NULL
        ptrs = list(full)
        ptrs[i] = None
        s, msg = _sa(p, ptrs)
        assert s == 1 and "NULL" in msg, i
    for i in range(9):                     # every pointer given must be 16-byte aligned
        ptrs = [ptr] * 9
        ptrs[i] = ctypes.c_void_p(24)
        assert _sa(p, ptrs)[0] == 4, i
    s, _ = _sa(_p(top_k=0), full)          # invalid problem
    assert s == 2
    pd = _p(q_len=1, kv_len=8192)          # decode needs the attention's workspace
    need = H.pyr_attn_workspace_bytes(pd)
    s, msg = _sa(pd, full)
    assert s == 5 and "workspace" in msg
    assert _sa(pd, full, ptr, need - 1)[0] == 5
    for kw in (dict(batch=0), dict(q_len=0, kv_len=0)):   # empty problems: nothing to do
        assert _sa(_p(**kw), [None] * 9)[0] == 0


def test_select_attn_binding_rejects_wrong_shapes_on_host():
    p = _p(q_len=128, kv_len=128)
    q = torch.zeros((1, 4, 128, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 128, 128), dtype=torch.bfloat16)
    pyr = torch.zeros(H.pyramid_shape(p))
    sel = torch.zeros((1, 2, 2, 9), dtype=torch.int32)
    with pytest.raises(ValueError):        # sel one slot short
        H.pyr_select_attn(p, q, k, k, pyr, sel[..., :8].contiguous(), q)
    with pytest.raises(ValueError):        # every shape right, but host tensors
        H.pyr_select_attn(p, q, k, k, pyr, sel, q)


def test_noalloc_validation_before_launch():
    """The allocation-free attention entry point validates like
    pyr_block_sparse_attn (minus the workspace) and refuses, before any HIP
    call, a problem whose partial states exceed its fixed scratch array."""
    ptr = ctypes.c_void_p(16)
    fn = "pyr_block_sparse_attn_noalloc"
    dec = _p(batch=512, n_q_heads=32, n_kv_heads=8, q_len=1, kv_len=4096, top_k=64)
    assert H.pyr_attn_workspace_bytes(dec) > 16 << 20
    s, msg = _status(fn, ctypes.byref(dec.c()), ptr, ptr, ptr, ptr, ptr, None, None)
    assert s == 5 and "16777216" in msg
    p = _p()
    for i in range(5):                     # q, k, v, sel, o may not be NULL
        ptrs = [ptr] * 5
        ptrs[i] = None
        assert _status(fn, ctypes.byref(p.c()), *ptrs, None, None)[0] == 1, i
    s, _ = _status(fn, ctypes.byref(p.c()), ptr, ptr, ptr, ptr, ptr, ctypes.c_void_p(20), None)
    assert s == 4
    bad = _p(head_dim=96)
    assert _status(fn, ctypes.byref(bad.c()), ptr, ptr, ptr, ptr, ptr, None, None)[0] == 3
