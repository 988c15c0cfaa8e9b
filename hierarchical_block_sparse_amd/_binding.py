"""ctypes binding of libpyr (include/pyr.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libpyr.so.  Tensors are torch tensors used as device memory; work goes on the
current torch stream unless a stream is given.  Each entry point checks on the
host that the tensors have the shapes, dtypes and device the problem implies,
so a kernel never sees a buffer smaller than its grid assumes.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PYR_LIBRARY names another build of the same library (the host-sanitizer build
# of hierarchical_block_sparse_amd.build, which the CPU ABI tests load).
LIB_PATH = os.environ.get("PYR_LIBRARY") or os.path.join(_HERE, "libpyr.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pyr.h")

PYR_F32, PYR_BF16 = 0, 1
ABI_VERSION = 5  # PYR_ABI_VERSION of the include/pyr.h these wrappers marshal for
STATUS = {0: "PYR_OK", 1: "PYR_ERR_NULL", 2: "PYR_ERR_INVALID", 3: "PYR_ERR_UNSUPPORTED",
          4: "PYR_ERR_MISALIGNED", 5: "PYR_ERR_WORKSPACE", 6: "PYR_ERR_HIP"}


class PyrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class PyrProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("block", ctypes.c_int32), ("branching", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("kv_capacity", ctypes.c_int64),
        ("cu", ctypes.c_void_p), ("total_len", ctypes.c_int64),
    ]


_lib_handle = None


def lib():
    """The loaded libpyr.so.  Raises if the HIP library has not been built: there
    is no fallback path."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hierarchical_block_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(PyrProblem)
        vp, st = ctypes.c_void_p, ctypes.c_int
        for name, res, args in [
            ("pyr_num_levels", ctypes.c_int32, [P]),
            ("pyr_level_offset", ctypes.c_int64, [P, ctypes.c_int32]),
            ("pyr_pyramid_nodes", ctypes.c_int64, [P]),
            ("pyr_pyramid_planes", ctypes.c_int32, [P]),
            ("pyr_num_query_blocks", ctypes.c_int64, [P]),
            ("pyr_attn_workspace_bytes", ctypes.c_size_t, [P]),
            ("pyr_build_pyramid", st, [P, vp, vp, vp]),
            ("pyr_append_pyramid", st, [P, vp, ctypes.c_int64, vp, vp]),
            ("pyr_select_topk", st, [P, vp, vp, vp, vp, vp, vp]),
            ("pyr_select_topk_budgets", st,
             [P, vp, vp, vp, ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp]),
            ("pyr_budgets_from_entropy", st,
             [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]),
            ("pyr_block_sparse_attn", st, [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
            ("pyr_block_sparse_attn_noalloc", st, [P, vp, vp, vp, vp, vp, vp, vp]),
            ("pyr_select_attn", st,
             [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
            ("pyr_attn_bwd_workspace_bytes", ctypes.c_size_t, [P]),
            ("pyr_block_sparse_attn_bwd", st,
             [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
            ("pyr_status_string", ctypes.c_char_p, [st]),
            ("pyr_last_error", ctypes.c_char_p, []),
            ("pyr_abi_version", ctypes.c_int32, []),
        ]:
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        if L.pyr_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.pyr_abi_version()}, these "
                               f"wrappers need {ABI_VERSION}: rebuild it")
        _lib_handle = L
    return _lib_handle


def declared_functions() -> list[str]:
    """Names of every function include/pyr.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pyr_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != 0:
        raise PyrError(status, lib().pyr_last_error().decode())


@dataclass(frozen=True)
class Problem:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    kv_len: int
    branching: int
    top_k: int
    dtype: torch.dtype
    scale: float = 0.0
    block: int = 64
    kv_capacity: int = 0  # 0: kv_len
    # packed sequences: int32 device tensor of batch+1 row offsets (None: dense)
    cu: torch.Tensor | None = field(default=None, compare=False, repr=False)
    total_len: int = 0    # packed: rows per head of q, k, v, o and lse

    def c(self) -> PyrProblem:
        code = {torch.float32: PYR_F32, torch.bfloat16: PYR_BF16}.get(self.dtype, 99)
        return PyrProblem(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.q_len,
                          self.kv_len, self.block, self.branching, self.top_k, code, self.scale,
                          self.kv_capacity, None if self.cu is None else self.cu.data_ptr(),
                          self.total_len)

    @property
    def packed(self) -> bool:
        return self.cu is not None

    @property
    def kv_rows(self) -> int:
        """Rows per head of k and v: the capacity, or kv_len (dense problems)."""
        return self.kv_capacity or self.kv_len

    @property
    def q_shape(self):
        """Shape of q and o: [B, Hq, q_len, d], packed [Hq, total_len, d]."""
        if self.packed:
            return (self.n_q_heads, self.total_len, self.head_dim)
        return (self.batch, self.n_q_heads, self.q_len, self.head_dim)

    @property
    def kv_shape(self):
        """Shape of k and v: [B, Hk, kv_rows, d], packed [Hk, total_len, d]."""
        if self.packed:
            return (self.n_kv_heads, self.total_len, self.head_dim)
        return (self.batch, self.n_kv_heads, self.kv_rows, self.head_dim)

    @property
    def lse_shape(self):
        return self.q_shape[:-1]

    @property
    def decode(self) -> bool:
        return self.q_len == 1 and self.kv_len > 1


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, shape, dtype, device_type="cuda"):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device.type != device_type:
        raise ValueError(f"{name}: must be a {device_type} tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _cp(p: Problem):
    """The C problem of p, after checking its packed-sequence offsets tensor."""
    if p.cu is not None:
        _expect(p.cu, "cu", (p.batch + 1,), torch.int32)
    return ctypes.byref(p.c())


# ---- geometry helpers (same names as the C ABI) ----

def pyr_num_levels(p: Problem) -> int:
    return lib().pyr_num_levels(ctypes.byref(p.c()))


def pyr_level_offset(p: Problem, level: int) -> int:
    return lib().pyr_level_offset(ctypes.byref(p.c()), level)


def pyr_pyramid_nodes(p: Problem) -> int:
    return lib().pyr_pyramid_nodes(ctypes.byref(p.c()))


def pyr_pyramid_planes(p: Problem) -> int:
    return lib().pyr_pyramid_planes(ctypes.byref(p.c()))


def pyramid_shape(p: Problem):
    """[B, Hk, planes, nodes, d]: the float32 pyramid buffer of a problem."""
    return (p.batch, p.n_kv_heads, pyr_pyramid_planes(p), pyr_pyramid_nodes(p), p.head_dim)


def pyr_num_query_blocks(p: Problem) -> int:
    return lib().pyr_num_query_blocks(ctypes.byref(p.c()))


def pyr_attn_workspace_bytes(p: Problem) -> int:
    return lib().pyr_attn_workspace_bytes(ctypes.byref(p.c()))


def pyr_abi_version() -> int:
    return lib().pyr_abi_version()


# ---- the hot path (same names as the C ABI) ----

def pyr_build_pyramid(p: Problem, k, pyramid, stream=None):
    _expect(k, "k", p.kv_shape, p.dtype)
    _expect(pyramid, "pyramid", pyramid_shape(p), torch.float32)
    _check(lib().pyr_build_pyramid(_cp(p), _ptr(k), _ptr(pyramid), _stream(stream)))


def pyr_append_pyramid(p: Problem, k, old_len: int, pyramid, stream=None):
    _expect(k, "k", p.kv_shape, p.dtype)
    _expect(pyramid, "pyramid", pyramid_shape(p), torch.float32)
    _check(lib().pyr_append_pyramid(_cp(p), _ptr(k), int(old_len), _ptr(pyramid),
                                    _stream(stream)))


def pyr_select_topk(p: Problem, q, pyramid, sel, trace_ids=None, trace_scores=None, stream=None):
    nqb, L = pyr_num_query_blocks(p), pyr_num_levels(p)
    _expect(q, "q", p.q_shape, p.dtype)
    _expect(pyramid, "pyramid", pyramid_shape(p), torch.float32)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(trace_ids, "trace_ids", (p.batch, p.n_kv_heads, nqb, L, p.top_k), torch.int32)
    _expect(trace_scores, "trace_scores", (p.batch, p.n_kv_heads, nqb, L, p.top_k + 1),
            torch.float32)
    _check(lib().pyr_select_topk(_cp(p), _ptr(q), _ptr(pyramid), _ptr(sel),
                                 _ptr(trace_ids), _ptr(trace_scores), _stream(stream)))


def pyr_select_topk_budgets(p: Problem, q, pyramid, sel, k_head=None, fallback_k: int = 0,
                            fallback_margin: float = 0.0, trace_ids=None, trace_scores=None,
                            stream=None):
    """Selection with per-KV-head budgets k_head (int32 [Hk] on the device, or
    None) and a finest-level confidence fallback to fallback_k blocks."""
    nqb, L = pyr_num_query_blocks(p), pyr_num_levels(p)
    _expect(q, "q", p.q_shape, p.dtype)
    _expect(pyramid, "pyramid", pyramid_shape(p), torch.float32)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(k_head, "k_head", (p.n_kv_heads,), torch.int32)
    _expect(trace_ids, "trace_ids", (p.batch, p.n_kv_heads, nqb, L, p.top_k), torch.int32)
    _expect(trace_scores, "trace_scores", (p.batch, p.n_kv_heads, nqb, L, p.top_k + 1),
            torch.float32)
    _check(lib().pyr_select_topk_budgets(_cp(p), _ptr(q), _ptr(pyramid), _ptr(k_head),
                                         int(fallback_k), float(fallback_margin), _ptr(sel),
                                         _ptr(trace_ids), _ptr(trace_scores), _stream(stream)))


def pyr_budgets_from_entropy(entropy, total: int, k_min: int, k_max: int) -> list[int]:
    """Per-head budgets in proportion to head entropy (host-only)."""
    n = len(entropy)
    ent = (ctypes.c_float * max(n, 1))(*[float(x) for x in entropy])
    out = (ctypes.c_int32 * max(n, 1))()
    _check(lib().pyr_budgets_from_entropy(ent, n, int(total), int(k_min), int(k_max), out))
    return [int(out[i]) for i in range(n)]


def pyr_block_sparse_attn(p: Problem, q, k, v, sel, o, lse=None, workspace=None, stream=None):
    nqb = pyr_num_query_blocks(p)
    _expect(q, "q", p.q_shape, p.dtype)
    _expect(k, "k", p.kv_shape, p.dtype)
    _expect(v, "v", p.kv_shape, p.dtype)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(o, "o", p.q_shape, p.dtype)
    _expect(lse, "lse", p.lse_shape, torch.float32)
    nbytes = 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace: must be a contiguous cuda tensor")
        nbytes = workspace.numel() * workspace.element_size()
    _check(lib().pyr_block_sparse_attn(_cp(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
                                       _ptr(o), _ptr(lse), _ptr(workspace), nbytes,
                                       _stream(stream)))


def pyr_block_sparse_attn_noalloc(p: Problem, q, k, v, sel, o, lse=None, stream=None):
    """pyr_block_sparse_attn without a workspace: the library's fixed
    per-device scratch array holds the decode partials (nothing is allocated)."""
    nqb = pyr_num_query_blocks(p)
    _expect(q, "q", p.q_shape, p.dtype)
    _expect(k, "k", p.kv_shape, p.dtype)
    _expect(v, "v", p.kv_shape, p.dtype)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(o, "o", p.q_shape, p.dtype)
    _expect(lse, "lse", p.lse_shape, torch.float32)
    _check(lib().pyr_block_sparse_attn_noalloc(_cp(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
                                               _ptr(o), _ptr(lse), _stream(stream)))


def pyr_select_attn(p: Problem, q, k, v, pyramid, sel, o, lse=None, workspace=None,
                    trace_ids=None, trace_scores=None, stream=None):
    """Selection and attention in one call (one fused launch where the library
    has one for the problem): writes sel (and the traces), o and lse."""
    nqb, L = pyr_num_query_blocks(p), pyr_num_levels(p)
    _expect(q, "q", p.q_shape, p.dtype)
    _expect(k, "k", p.kv_shape, p.dtype)
    _expect(v, "v", p.kv_shape, p.dtype)
    _expect(pyramid, "pyramid", pyramid_shape(p), torch.float32)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(trace_ids, "trace_ids", (p.batch, p.n_kv_heads, nqb, L, p.top_k), torch.int32)
    _expect(trace_scores, "trace_scores", (p.batch, p.n_kv_heads, nqb, L, p.top_k + 1),
            torch.float32)
    _expect(o, "o", p.q_shape, p.dtype)
    _expect(lse, "lse", p.lse_shape, torch.float32)
    nbytes = 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace: must be a contiguous cuda tensor")
        nbytes = workspace.numel() * workspace.element_size()
    _check(lib().pyr_select_attn(_cp(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pyramid), _ptr(sel),
                                 _ptr(trace_ids), _ptr(trace_scores), _ptr(o), _ptr(lse),
                                 _ptr(workspace), nbytes, _stream(stream)))


def pyr_attn_bwd_workspace_bytes(p: Problem) -> int:
    return lib().pyr_attn_bwd_workspace_bytes(_cp(p))


def _workspace_bytes(workspace) -> int:
    if workspace is None:
        return 0
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous cuda tensor")
    return workspace.numel() * workspace.element_size()


def pyr_block_sparse_attn_bwd(p: Problem, q, k, v, sel, o, lse, dout, dq, dk, dv, workspace,
                              stream=None):
    nqb = pyr_num_query_blocks(p)
    qs = p.q_shape
    ks = p.kv_shape
    for t, name, shape in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (o, "o", qs),
                           (dout, "dout", qs), (dq, "dq", qs), (dk, "dk", ks), (dv, "dv", ks)):
        _expect(t, name, shape, p.dtype)
    _expect(sel, "sel", (p.batch, p.n_kv_heads, nqb, p.top_k + 1), torch.int32)
    _expect(lse, "lse", p.lse_shape, torch.float32)
    _check(lib().pyr_block_sparse_attn_bwd(
        _cp(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(o), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _workspace_bytes(workspace),
        _stream(stream)))


# ---- allocating conveniences (torch allocates; the library computes) ----

def alloc_pyramid(p: Problem, device="cuda"):
    return torch.empty(pyramid_shape(p), dtype=torch.float32, device=device)


def alloc_sel(p: Problem, device="cuda"):
    return torch.empty((p.batch, p.n_kv_heads, pyr_num_query_blocks(p), p.top_k + 1),
                       dtype=torch.int32, device=device)


def alloc_trace(p: Problem, device="cuda"):
    nqb, L = pyr_num_query_blocks(p), pyr_num_levels(p)
    ids = torch.empty((p.batch, p.n_kv_heads, nqb, L, p.top_k), dtype=torch.int32, device=device)
    sc = torch.empty((p.batch, p.n_kv_heads, nqb, L, p.top_k + 1), dtype=torch.float32,
                     device=device)
    return ids, sc


def alloc_workspace(p: Problem, device="cuda"):
    n = pyr_attn_workspace_bytes(p)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def alloc_bwd_workspace(p: Problem, device="cuda"):
    n = pyr_attn_bwd_workspace_bytes(p)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def backward(q, k, v, sel, o, lse, dout, branching: int, top_k: int, scale: float = 0.0):
    """dq, dk, dv of the attention for the forward's route rows (fixed routes)."""
    p = problem_for(q, k, branching, top_k, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pyr_block_sparse_attn_bwd(p, q, k, v, sel, o, lse, dout, dq, dk, dv,
                              alloc_bwd_workspace(p, q.device))
    return dq, dk, dv


def problem_for(q, k, branching: int, top_k: int, scale: float = 0.0) -> Problem:
    B, Hq, Tq, d = q.shape
    _, Hk, Tk, _ = k.shape
    return Problem(B, Hq, Hk, d, Tq, Tk, branching, top_k, q.dtype, scale)


def forward(q, k, v, branching: int, top_k: int, scale: float = 0.0, pyramid=None,
            with_trace: bool = False, fused: bool = False):
    """The whole path: build the pyramid (unless given), select, attend (with
    fused=True, selection and attention in one pyr_select_attn call).
    Returns (o, lse, sel, pyramid[, (trace_ids, trace_scores)])."""
    p = problem_for(q, k, branching, top_k, scale)
    if pyramid is None:
        pyramid = alloc_pyramid(p, q.device)
        pyr_build_pyramid(p, k, pyramid)
    sel = alloc_sel(p, q.device)
    trace = alloc_trace(p, q.device) if with_trace else (None, None)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if fused:
        pyr_select_attn(p, q, k, v, pyramid, sel, o, lse, alloc_workspace(p, q.device), *trace)
    else:
        pyr_select_topk(p, q, pyramid, sel, *trace)
        pyr_block_sparse_attn(p, q, k, v, sel, o, lse, alloc_workspace(p, q.device))
    if with_trace:
        return o, lse, sel, pyramid, trace
    return o, lse, sel, pyramid


def problem_for_packed(q, k, cu, max_len: int, branching: int, top_k: int,
                       scale: float = 0.0) -> Problem:
    """The packed problem of q [Hq, total, d], k [Hk, total, d] and row offsets
    cu (int32, batch+1 entries) whose sequences are at most max_len long."""
    Hq, total, d = q.shape
    Hk = k.shape[0]
    return Problem(cu.numel() - 1, Hq, Hk, d, max_len, max_len, branching, top_k, q.dtype, scale,
                   cu=cu, total_len=total)


def forward_packed(q, k, v, cu, max_len: int, branching: int, top_k: int, scale: float = 0.0):
    """The whole path on a packed batch: every sequence attends within itself.
    Returns (o, lse, sel, pyramid) with o like q and lse [Hq, total]; rows of
    no sequence are left as torch.empty leaves them."""
    p = problem_for_packed(q, k, cu, max_len, branching, top_k, scale)
    pyramid = alloc_pyramid(p, q.device)
    pyr_build_pyramid(p, k, pyramid)
    sel = alloc_sel(p, q.device)
    pyr_select_topk(p, q, pyramid, sel)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    pyr_block_sparse_attn(p, q, k, v, sel, o, lse, alloc_workspace(p, q.device))
    return o, lse, sel, pyramid
