"""newton_schulz_gram_amd — batched Newton–Schulz / Gram Newton–Schulz on MI355X.

A thin ctypes binding over libnsg.so (include/nsg.h).  Every step of the
orthogonalization runs in the library's gfx950 HIP kernels; this module only
checks and marshals arguments, takes device memory and the current stream from
PyTorch, and raises if the library is missing or a call fails.  There is no
CPU fallback.

    import torch, newton_schulz_gram_amd as nsg
    O = nsg.orthogonalize(G)            # G: [R, C] or [G, R, C] on the GPU
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsg.so")

NSG_F16, NSG_BF16, NSG_F32 = 0, 1, 2
NSG_STANDARD, NSG_GRAM = 0, 1
MUON_COEFFS = (3.4445, -4.7750, 2.0315)  # "muon" kernel card, "How it works"

_DT = {torch.float16: NSG_F16, torch.bfloat16: NSG_BF16, torch.float32: NSG_F32}
_DT_NAMES = {"f16": NSG_F16, "fp16": NSG_F16, "float16": NSG_F16,
             "bf16": NSG_BF16, "bfloat16": NSG_BF16,
             "f32": NSG_F32, "fp32": NSG_F32, "float32": NSG_F32}
_MODES = {"standard": NSG_STANDARD, "gram": NSG_GRAM}
KIND_NAMES = {0: "norm_reduce", 1: "scale_cast_transpose", 2: "gemm_nt", 3: "gemm_nt_sym"}

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype", 3: "unsupported shape",
          4: "workspace missing, misaligned or too small", 5: "HIP runtime error",
          6: "bucket needs more than the fixed no-allocation scratch"}
NOALLOC_MAX_BYTES = 128 << 20  # NSG_NOALLOC_MAX_BYTES


class NSGError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, 'status %d' % code)} (nsg status {code})")
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [
        ("steps", ctypes.c_int32),
        ("coeffs", ctypes.POINTER(ctypes.c_double)),
        ("n_coeffs", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("restart_after", ctypes.c_int32),
        ("safety", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("compute_dtype", ctypes.c_int32),
        ("sym_updates", ctypes.c_int32),
        ("restart_mask", ctypes.c_uint64),
    ]


class LaunchInfo(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("step", ctypes.c_int32),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
        ("label", ctypes.c_char * 24),
        ("a_kmajor", ctypes.c_int32),
        ("b_kmajor", ctypes.c_int32),
        ("source", ctypes.c_int32),
    ]


# nsg_launch_info_t.source: where a GEMM's operands come from
SOURCE_NAMES = {0: "plain", 1: "A converted from bf16", 2: "B converted from bf16", 3: "raw bf16"}


EXPORTS = ("ns_default_params", "ns_workspace_size", "ns_orthogonalize", "ns_status_string",
           "ns_flops", "ns_plan", "ns_timing_enable", "ns_timing_collect", "nsg_copy",
           "nsg_gemm_nt", "ns_select_workspace_size", "ns_orthogonalize_selected",
           "nsg_l1_workspace_size", "nsg_l1_norms", "nsg_topk", "ns_muon_momentum", "ns_muon_update",
           "ns_muon_workspace_size", "ns_muon_step", "ns_select_count", "ns_orthogonalize_noalloc")
SELECT_ROWS, SELECT_COLS, SELECT_SMALLER = 0, 1, -1

_lib = None


def lib() -> ctypes.CDLL:
    """Load libnsg.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libnsg.so is not built ({LIB_PATH}); run "
                           "`python -m newton_schulz_gram_amd.build` or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(Params)
    L.ns_default_params.argtypes = [P]
    L.ns_default_params.restype = None
    L.ns_workspace_size.argtypes = [i64, i64, i64, P, ctypes.POINTER(sz)]
    L.ns_workspace_size.restype = i32
    L.ns_orthogonalize.argtypes = [vp, i32, vp, i32, i64, i64, i64, P, vp, sz, vp, vp]
    L.ns_orthogonalize.restype = i32
    L.ns_orthogonalize_noalloc.argtypes = [vp, i32, vp, i32, i64, i64, i64, P, vp, vp]
    L.ns_orthogonalize_noalloc.restype = i32
    L.ns_status_string.argtypes = [i32]
    L.ns_status_string.restype = ctypes.c_char_p
    L.ns_flops.argtypes = [i64, i64, P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.ns_flops.restype = i32
    L.ns_plan.argtypes = [i64, i64, i32, P, ctypes.POINTER(LaunchInfo), i32, ctypes.POINTER(i32)]
    L.ns_plan.restype = i32
    L.ns_timing_enable.argtypes = [i32]
    L.ns_timing_enable.restype = i32
    L.ns_timing_collect.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(f32), i32, ctypes.POINTER(i32)]
    L.ns_timing_collect.restype = i32
    L.nsg_copy.argtypes = [vp, vp, sz, vp]
    L.nsg_copy.restype = i32
    L.nsg_gemm_nt.argtypes = [i32, i32, i64, i64, i64, i64, vp, i64, i32, vp, i64, i32, f32, f32, vp, i64,
                              vp, i64, vp, i64, vp, f32, i32, vp, vp]
    L.nsg_gemm_nt.restype = i32
    L.ns_select_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32, i32, P, ctypes.POINTER(sz)]
    L.ns_select_workspace_size.restype = i32
    L.ns_orthogonalize_selected.argtypes = [vp, i32, vp, i32, i64, i64, i64, i64, i32, P, vp, sz, vp, vp, vp]
    L.ns_orthogonalize_selected.restype = i32
    L.ns_select_count.argtypes = [i64, i64, i32, ctypes.c_double, ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.ns_select_count.restype = i32
    L.nsg_l1_workspace_size.argtypes = [i64, i64, i64, i32, ctypes.POINTER(sz)]
    L.nsg_l1_workspace_size.restype = i32
    L.nsg_l1_norms.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, sz, vp]
    L.nsg_l1_norms.restype = i32
    L.nsg_topk.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    L.nsg_topk.restype = i32
    f64, u64 = ctypes.c_double, ctypes.c_uint64
    L.ns_muon_momentum.argtypes = [vp, i32, vp, i32, i64, f32, vp]
    L.ns_muon_momentum.restype = i32
    L.ns_muon_update.argtypes = [vp, i32, vp, i32, i64, f64, f64, f64, i32, u64, u64, vp]
    L.ns_muon_update.restype = i32
    L.ns_muon_workspace_size.argtypes = [i64, i64, i64, P, ctypes.POINTER(sz)]
    L.ns_muon_workspace_size.restype = i32
    L.ns_muon_step.argtypes = [vp, i32, vp, i32, vp, i32, i64, i64, i64, f32, f64, f64, f64, i32, u64, u64, P,
                               vp, sz, vp, vp]
    L.ns_muon_step.restype = i32
    _lib = L
    return L


def _check(code: int, what: str):
    if code != 0:
        raise NSGError(code, what)


def _dtype_code(dt) -> int:
    if isinstance(dt, str):
        return _DT_NAMES[dt]
    if isinstance(dt, torch.dtype):
        if dt not in _DT:
            raise TypeError(f"unsupported dtype {dt}")
        return _DT[dt]
    return int(dt)


def make_params(steps: int = 5, coeffs: Optional[Sequence[float]] = None, mode: str = "gram",
                restart_after: int = 2, safety: float = 1.05, eps: float = 1e-7,
                compute_dtype="f16", sym_updates: bool = True, restarts: Optional[Sequence[int]] = None):
    """Build an nsg_params_t.  Returns (params, keepalive) — keep both alive.

    `restarts` lists the steps t (2..steps) at whose top the Gram iteration
    restarts; it overrides `restart_after` (a single restart)."""
    c = list(MUON_COEFFS if coeffs is None else coeffs)
    arr = (ctypes.c_double * len(c))(*[float(x) for x in c])
    p = Params()
    p.steps = int(steps)
    p.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_double))
    p.n_coeffs = len(c)
    p.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    p.restart_after = int(restart_after)
    p.safety = float(safety)
    p.eps = float(eps)
    p.compute_dtype = _dtype_code(compute_dtype)
    p.sym_updates = 1 if sym_updates else 0
    mask = 0
    for t in (restarts or ()):
        t = int(t)
        if not 1 <= t <= 64:
            raise ValueError("restart steps must lie in 2..steps")
        mask |= 1 << (t - 1)
    p.restart_mask = mask
    return p, arr


def workspace_size(G: int, R: int, C: int, **kw) -> int:
    p, _keep = make_params(**kw)
    out = ctypes.c_size_t(0)
    _check(lib().ns_workspace_size(G, R, C, ctypes.byref(p), ctypes.byref(out)), "ns_workspace_size")
    return int(out.value)


def flops(R: int, C: int, **kw):
    """(credited, executed) FLOPs per matrix (the pages' formula; the plan's tiles)."""
    p, _keep = make_params(**kw)
    cr, ex = ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().ns_flops(R, C, ctypes.byref(p), ctypes.byref(cr), ctypes.byref(ex)), "ns_flops")
    return cr.value, ex.value


def plan(R: int, C: int, in_dtype=None, **kw):
    """The launch list of one call on an input of dtype `in_dtype` (default:
    the compute dtype), as a list of dicts (host only)."""
    p, _keep = make_params(**kw)
    idt = p.compute_dtype if in_dtype is None else _dtype_code(in_dtype)
    n = ctypes.c_int32(0)
    _check(lib().ns_plan(R, C, idt, ctypes.byref(p), None, 0, ctypes.byref(n)), "ns_plan")
    arr = (LaunchInfo * max(1, n.value))()
    _check(lib().ns_plan(R, C, idt, ctypes.byref(p), arr, n.value, ctypes.byref(n)), "ns_plan")
    return [dict(kind=e.kind, kernel=KIND_NAMES[e.kind], step=e.step, M=e.M, N=e.N, K=e.K,
                 flops=e.flops, bytes=e.bytes, label=e.label.decode(), a_kmajor=bool(e.a_kmajor),
                 b_kmajor=bool(e.b_kmajor), source=e.source) for e in arr[:n.value]]


def nbytes(t: torch.Tensor) -> int:
    """Bytes of a tensor's storage as the library sees it (numel x element size)."""
    return t.numel() * t.element_size()


def check_out(out: torch.Tensor, nb: int, R: int, C: int, squeeze: bool, device) -> None:
    """A caller-supplied output must hold exactly the bucket: [nb, R, C], or
    [R, C] when the input was one 2-D matrix; contiguous, on the input's device.
    The library writes nb * R * C elements into it."""
    ok_shape = tuple(out.shape) == (nb, R, C) or (squeeze and nb == 1 and tuple(out.shape) == (R, C))
    if not ok_shape:
        raise ValueError(f"out has shape {tuple(out.shape)}; expected {(R, C) if squeeze else (nb, R, C)}")
    if out.dtype not in _DT:
        raise ValueError(f"unsupported out dtype {out.dtype}")
    if not out.is_contiguous() or out.device != device:
        raise ValueError("out must be contiguous on the input's device")


def check_workspace(ws: torch.Tensor, device) -> None:
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the input's device")


def check_status(status: Optional[torch.Tensor], nb: int, device) -> None:
    """status: None, or int32 with at least nb entries, contiguous, on the input's device."""
    if status is None:
        return
    if status.dtype != torch.int32 or status.numel() < nb or not status.is_contiguous() or status.device != device:
        raise ValueError("status must be a contiguous int32 tensor with G entries on the input's device")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def orthogonalize(G: torch.Tensor, steps: int = 5, coeffs: Optional[Sequence[float]] = None,
                  mode: str = "gram", restart_after: int = 2, safety: float = 1.05,
                  eps: float = 1e-7, compute_dtype="f16", out_dtype=None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  status: Optional[torch.Tensor] = None, sym_updates: bool = True,
                  restarts: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Orthogonalize one matrix [R, C] or a bucket [G, R, C] on its GPU.

    sym_updates (default) runs Q Z + a Q and R Z + a R on the symmetric kernel
    (Gram mode; half the tiles, exactly symmetric results); False runs them
    as general products.  `restarts` lists several restart steps (see
    make_params).

    Returns `out` (allocated if not given) with dtype out_dtype (default: the
    input's).  `status`, if given, is an int32 CUDA tensor of G entries set to
    1 for matrices whose output has a non-finite value.
    """
    if not G.is_cuda:
        raise ValueError("orthogonalize needs a GPU tensor (no CPU path)")
    squeeze = G.dim() == 2
    Gs = G.unsqueeze(0) if squeeze else G
    if Gs.dim() != 3:
        raise ValueError("expected [R, C] or [G, R, C]")
    if not Gs.is_contiguous():
        raise ValueError("input must be contiguous")
    nb, R, C = Gs.shape
    odt = Gs.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((nb, R, C), dtype=odt, device=Gs.device)
    else:
        check_out(out, nb, R, C, squeeze, Gs.device)
        odt = out.dtype
    p, _keep = make_params(steps, coeffs, mode, restart_after, safety, eps, compute_dtype, sym_updates,
                           restarts)
    need = ctypes.c_size_t(0)
    _check(lib().ns_workspace_size(nb, R, C, ctypes.byref(p), ctypes.byref(need)), "ns_workspace_size")
    if workspace is None or nbytes(workspace) < need.value:
        workspace = torch.empty(max(1, need.value), dtype=torch.uint8, device=Gs.device)
    check_workspace(workspace, Gs.device)
    check_status(status, nb, Gs.device)
    with torch.cuda.device(Gs.device):
        code = lib().ns_orthogonalize(
            ctypes.c_void_p(Gs.data_ptr()), _dtype_code(Gs.dtype),
            ctypes.c_void_p(out.data_ptr()), _dtype_code(odt),
            nb, R, C, ctypes.byref(p),
            ctypes.c_void_p(workspace.data_ptr()), nbytes(workspace),
            ctypes.c_void_p(status.data_ptr()) if status is not None else None,
            ctypes.c_void_p(_stream_handle(Gs.device)))
    _check(code, "ns_orthogonalize")
    return out[0] if (squeeze and out.dim() == 3) else out


def orthogonalize_noalloc(G: torch.Tensor, out: torch.Tensor, steps: int = 5,
                          coeffs: Optional[Sequence[float]] = None, mode: str = "gram", restart_after: int = 2,
                          safety: float = 1.05, eps: float = 1e-7, compute_dtype="f16",
                          status: Optional[torch.Tensor] = None, sym_updates: bool = True,
                          restarts: Optional[Sequence[int]] = None) -> torch.Tensor:
    """orthogonalize() through ns_orthogonalize_noalloc: the library's fixed
    scratch array is the workspace, so neither the library nor this wrapper
    allocates device memory (the caller passes `out`).  Buckets whose
    workspace exceeds NOALLOC_MAX_BYTES raise NSGError (status 6).  Calls that
    may overlap on one GPU share that scratch and race."""
    if not G.is_cuda:
        raise ValueError("orthogonalize_noalloc needs a GPU tensor (no CPU path)")
    squeeze = G.dim() == 2
    Gs = G.unsqueeze(0) if squeeze else G
    if Gs.dim() != 3 or not Gs.is_contiguous():
        raise ValueError("expected a contiguous [R, C] or [G, R, C] tensor")
    nb, R, C = Gs.shape
    check_out(out, nb, R, C, squeeze, Gs.device)
    check_status(status, nb, Gs.device)
    p, _keep = make_params(steps, coeffs, mode, restart_after, safety, eps, compute_dtype, sym_updates, restarts)
    with torch.cuda.device(Gs.device):
        code = lib().ns_orthogonalize_noalloc(
            ctypes.c_void_p(Gs.data_ptr()), _dtype_code(Gs.dtype), ctypes.c_void_p(out.data_ptr()),
            _dtype_code(out.dtype), nb, R, C, ctypes.byref(p),
            ctypes.c_void_p(status.data_ptr()) if status is not None else None,
            ctypes.c_void_p(_stream_handle(Gs.device)))
    _check(code, "ns_orthogonalize_noalloc")
    return out


def timing_enable(on: bool = True):
    _check(lib().ns_timing_enable(1 if on else 0), "ns_timing_enable")


def timing_collect(max_entries: int = 1 << 16):
    """[(kernel name, ms), ...] for every launch recorded since the last collect."""
    kinds = (ctypes.c_int32 * max_entries)()
    ms = (ctypes.c_float * max_entries)()
    n = ctypes.c_int32(0)
    _check(lib().ns_timing_collect(kinds, ms, max_entries, ctypes.byref(n)), "ns_timing_collect")
    return [(KIND_NAMES[kinds[i]], float(ms[i])) for i in range(min(n.value, max_entries))]


def copy(src: torch.Tensor, dst: torch.Tensor):
    """Library copy kernel (byte-counter calibration)."""
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        _check(lib().nsg_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                              ctypes.c_void_p(_stream_handle(src.device))), "nsg_copy")


def gemm_nt(A: torch.Tensor, B: torch.Tensor, alpha: float = 1.0, beta: float = 0.0,
            Cin: Optional[torch.Tensor] = None, symmetric: bool = False, transposed_out: bool = False,
            diag: Optional[float] = None, tile: int = 0, a_kmajor: bool = False, b_kmajor: bool = False,
            status: Optional[torch.Tensor] = None):
    """Library GEMM building block: V = alpha A B^T + beta Cin over a batch.

    A [b, M, K], B [b, N, K] (M, N, K multiples of 256) in one dtype; tile 128
    or 256 picks the kernel (0: the library's choice).  With a_kmajor
    (b_kmajor) A (B) is passed K-major instead, as [b, K, M] ([b, K, N]).
    Returns (V, V^T or None, V + diag I or None)."""
    b = A.shape[0]
    M, K = (A.shape[2], A.shape[1]) if a_kmajor else (A.shape[1], A.shape[2])
    N = B.shape[2] if b_kmajor else B.shape[1]
    for t in (A, B) + ((Cin,) if Cin is not None else ()):
        if t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError("gemm_nt operands need unit column stride and packed batches")
    out = torch.empty((b, M, N), dtype=A.dtype, device=A.device)
    out_t = torch.empty((b, N, M), dtype=A.dtype, device=A.device) if transposed_out else None
    out_d = torch.empty((b, M, N), dtype=A.dtype, device=A.device) if diag is not None else None
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    with torch.cuda.device(A.device):
        code = lib().nsg_gemm_nt(_dtype_code(A.dtype), 1 if symmetric else 0, b, M, N, K,
                                 ptr(A), A.stride(1), 1 if a_kmajor else 0, ptr(B), B.stride(1),
                                 1 if b_kmajor else 0, float(alpha), float(beta), ptr(Cin),
                                 Cin.stride(1) if Cin is not None else N,
                                 ptr(out), N, ptr(out_t), M, ptr(out_d), float(diag or 0.0), int(tile), ptr(status),
                                 ctypes.c_void_p(_stream_handle(A.device)))
    _check(code, "nsg_gemm_nt")
    return out, out_t, out_d


# ---------------------------------------------------------------------------
# Dion3 selection front-end (Dion3 paper, Section 6; Algorithm 4, steps 3-4)
# ---------------------------------------------------------------------------

def select_plan(R: int, C: int, fraction: float, dim: int = SELECT_SMALLER):
    """(resolved dim, k) of the library's selection rule: k = ceil(f n) lines
    of rows (dim 0) or columns (dim 1); -1 picks the smaller dimension."""
    d, k = ctypes.c_int32(0), ctypes.c_int64(0)
    code = lib().ns_select_count(int(R), int(C), int(dim), float(fraction), ctypes.byref(d), ctypes.byref(k))
    if code == 1:
        raise ValueError("fraction must lie in (0, 1] and dim in {-1, 0, 1}")
    _check(code, "ns_select_count")
    return int(d.value), int(k.value)


def select_count(n: int, fraction: float) -> int:
    """k = ceil(f n) lines out of n (at least 1), by the library's rule."""
    return select_plan(n, n, fraction, SELECT_ROWS)[1]


def orthogonalize_selected(M: torch.Tensor, fraction: float = 0.25, k: Optional[int] = None, dim: int = -1,
                           steps: int = 5, coeffs: Optional[Sequence[float]] = None, mode: str = "gram",
                           restart_after: int = 2, safety: float = 1.05, eps: float = 1e-7,
                           compute_dtype="f16", out_dtype=None, out: Optional[torch.Tensor] = None,
                           status: Optional[torch.Tensor] = None, sym_updates: bool = True,
                           restarts: Optional[Sequence[int]] = None):
    """Select the k = ceil(f n) rows (dim 0) or columns (dim 1; -1: the smaller
    dimension) of largest l1 norm of every matrix, orthogonalize them, and
    return (out, idx): out [G, R, C] holds the result in the selected lines and
    zeros elsewhere, idx [G, k] int32 the selected indices (ascending)."""
    if not M.is_cuda:
        raise ValueError("orthogonalize_selected needs a GPU tensor (no CPU path)")
    squeeze = M.dim() == 2
    Ms = M.unsqueeze(0) if squeeze else M
    if Ms.dim() != 3 or not Ms.is_contiguous():
        raise ValueError("expected a contiguous [R, C] or [G, R, C] tensor")
    G, R, C = Ms.shape
    if k is None:
        d, kk = select_plan(R, C, fraction, dim)
    else:
        d, _ = select_plan(R, C, 1.0, dim)
        kk = int(k)
    odt = Ms.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((G, R, C), dtype=odt, device=Ms.device)
    else:
        check_out(out, G, R, C, squeeze, Ms.device)
    odt = out.dtype
    check_status(status, G, Ms.device)
    idx = torch.empty((G, kk), dtype=torch.int32, device=Ms.device)
    p, _keep = make_params(steps, coeffs, mode, restart_after, safety, eps, compute_dtype, sym_updates, restarts)
    need = ctypes.c_size_t(0)
    _check(lib().ns_select_workspace_size(G, R, C, kk, d, _dtype_code(Ms.dtype), _dtype_code(odt), ctypes.byref(p),
                                          ctypes.byref(need)), "ns_select_workspace_size")
    ws = torch.empty(max(1, need.value), dtype=torch.uint8, device=Ms.device)
    with torch.cuda.device(Ms.device):
        _check(lib().ns_orthogonalize_selected(
            ctypes.c_void_p(Ms.data_ptr()), _dtype_code(Ms.dtype), ctypes.c_void_p(out.data_ptr()), _dtype_code(odt),
            G, R, C, kk, d, ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), need.value,
            ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(status.data_ptr()) if status is not None else None,
            ctypes.c_void_p(_stream_handle(Ms.device))), "ns_orthogonalize_selected")
    if squeeze:
        return out[0], idx[0]
    return out, idx


def l1_norms(M: torch.Tensor, dim: int = 0) -> torch.Tensor:
    """fp64 l1 norms of the rows (dim 0) or columns (dim 1) of [G, R, C]."""
    Ms = M.unsqueeze(0) if M.dim() == 2 else M
    if not Ms.is_contiguous():
        raise ValueError("input must be contiguous")
    G, R, C = Ms.shape
    n = R if dim == SELECT_ROWS else C
    keys = torch.empty((G, n), dtype=torch.float64, device=Ms.device)
    need = ctypes.c_size_t(0)
    _check(lib().nsg_l1_workspace_size(G, R, C, dim, ctypes.byref(need)), "nsg_l1_workspace_size")
    ws = torch.empty(max(1, need.value), dtype=torch.uint8, device=Ms.device)
    with torch.cuda.device(Ms.device):
        _check(lib().nsg_l1_norms(ctypes.c_void_p(Ms.data_ptr()), _dtype_code(Ms.dtype), G, R, C, dim,
                                  ctypes.c_void_p(keys.data_ptr()), ctypes.c_void_p(ws.data_ptr()), need.value,
                                  ctypes.c_void_p(_stream_handle(Ms.device))), "nsg_l1_norms")
    return keys


def topk(keys: torch.Tensor, k: int):
    """(idx [G, k] ascending, pos [G, n]) of the k largest keys per row of keys."""
    keys = keys.contiguous().to(torch.float64)
    G, n = keys.shape
    idx = torch.empty((G, k), dtype=torch.int32, device=keys.device)
    pos = torch.empty((G, n), dtype=torch.int32, device=keys.device)
    with torch.cuda.device(keys.device):
        _check(lib().nsg_topk(ctypes.c_void_p(keys.data_ptr()), G, n, k, ctypes.c_void_p(idx.data_ptr()),
                              ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(_stream_handle(keys.device))),
               "nsg_topk")
    return idx, pos


# ---------------------------------------------------------------------------
# The Muon step (Dion3 paper, Eq. (1); Algorithm 4, steps 8-9; muon card)
# ---------------------------------------------------------------------------

def muon_momentum(M: torch.Tensor, G: torch.Tensor, mu: float):
    """In place: M <- mu M + G (fp32 arithmetic; M is float32 or bfloat16)."""
    if M.numel() != G.numel() or not (M.is_contiguous() and G.is_contiguous()):
        raise ValueError("M and G must be contiguous with the same number of elements")
    with torch.cuda.device(M.device):
        _check(lib().ns_muon_momentum(ctypes.c_void_p(M.data_ptr()), _dtype_code(M.dtype), ctypes.c_void_p(G.data_ptr()),
                                      _dtype_code(G.dtype), M.numel(), float(mu),
                                      ctypes.c_void_p(_stream_handle(M.device))), "ns_muon_momentum")
    return M


def muon_update(W: torch.Tensor, O: torch.Tensor, lr: float, weight_decay: float = 0.0, scale: float = 1.0,
                stochastic: bool = True, seed: int = 0, step: int = 0):
    """In place: W <- (1 - lr wd) W - lr scale O; a bf16 W is written back with
    counter-based stochastic rounding (seed, step, element index)."""
    if W.numel() != O.numel() or not (W.is_contiguous() and O.is_contiguous()):
        raise ValueError("W and O must be contiguous with the same number of elements")
    with torch.cuda.device(W.device):
        _check(lib().ns_muon_update(ctypes.c_void_p(W.data_ptr()), _dtype_code(W.dtype), ctypes.c_void_p(O.data_ptr()),
                                    _dtype_code(O.dtype), W.numel(), float(lr), float(weight_decay), float(scale),
                                    1 if stochastic else 0, int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1),
                                    ctypes.c_void_p(_stream_handle(W.device))), "ns_muon_update")
    return W


def muon_step(W: torch.Tensor, M: torch.Tensor, G: torch.Tensor, mu: float, lr: float, weight_decay: float = 0.0,
              scale: float = 1.0, stochastic: bool = True, seed: int = 0, step: int = 0,
              status: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, **kw):
    """One Muon step for a bucket [G, R, C] (or one [R, C] matrix), in place on
    W and M; keyword arguments set the Newton-Schulz parameters."""
    Ws, Ms, Gs = (t.unsqueeze(0) if t.dim() == 2 else t for t in (W, M, G))
    if not (Ws.shape == Ms.shape == Gs.shape) or Ws.dim() != 3:
        raise ValueError("W, M and G must share a [G, R, C] or [R, C] shape")
    if not (Ws.is_contiguous() and Ms.is_contiguous() and Gs.is_contiguous()):
        raise ValueError("W, M and G must be contiguous")
    nb, R, C = Ws.shape
    p, _keep = make_params(**kw)
    need = ctypes.c_size_t(0)
    _check(lib().ns_muon_workspace_size(nb, R, C, ctypes.byref(p), ctypes.byref(need)), "ns_muon_workspace_size")
    if workspace is None or nbytes(workspace) < need.value:
        workspace = torch.empty(max(1, need.value), dtype=torch.uint8, device=Ws.device)
    if not (Ms.device == Gs.device == Ws.device):
        raise ValueError("W, M and G must be on one device")
    check_workspace(workspace, Ws.device)
    check_status(status, nb, Ws.device)
    with torch.cuda.device(Ws.device):
        _check(lib().ns_muon_step(
            ctypes.c_void_p(Ws.data_ptr()), _dtype_code(Ws.dtype), ctypes.c_void_p(Ms.data_ptr()), _dtype_code(Ms.dtype),
            ctypes.c_void_p(Gs.data_ptr()), _dtype_code(Gs.dtype), nb, R, C, float(mu), float(lr), float(weight_decay),
            float(scale), 1 if stochastic else 0, int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1), ctypes.byref(p),
            ctypes.c_void_p(workspace.data_ptr()), nbytes(workspace),
            ctypes.c_void_p(status.data_ptr()) if status is not None else None,
            ctypes.c_void_p(_stream_handle(Ws.device))), "ns_muon_step")
    return W, M
