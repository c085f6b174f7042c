"""CPU tests of the C-ABI library: it loads, exports every symbol include/nsg.h
declares, validates arguments before touching the GPU, and its planner's FLOP
tally matches the pages' formulas (no GPU needed for any of this)."""
import ctypes
import os
import re

import pytest

import newton_schulz_gram_amd as nsg
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsg.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:nsg_status_t|void|const char \*)\s*\n?\s*(\w+)\s*\(", text,
                                 flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = nsg.lib()
    names = header_functions()
    assert len(names) >= 10, names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(nsg.EXPORTS)


def test_status_strings():
    L = nsg.lib()
    for code in range(7):
        assert L.ns_status_string(code).decode() == nsg.STATUS[code]


def test_default_params():
    p = nsg.Params()
    nsg.lib().ns_default_params(ctypes.byref(p))
    assert p.steps == 5 and p.n_coeffs == 3 and p.mode == nsg.NSG_GRAM
    assert p.restart_after == 2 and abs(p.safety - 1.05) < 1e-6 and abs(p.eps - 1e-7) < 1e-12
    assert [p.coeffs[i] for i in range(3)] == list(nsg.MUON_COEFFS)
    assert p.compute_dtype == nsg.NSG_F16
    assert p.sym_updates == 1


def _call(G=2, R=64, C=128, in_dtype=0, out_dtype=0, ws_bytes=None, ws_ptr=1 << 20, **kw):
    p, keep = nsg.make_params(**kw)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    # fake device pointers: validation must fail before anything dereferences them
    return nsg.lib().ns_orthogonalize(ctypes.c_void_p(0x1000), in_dtype, ctypes.c_void_p(0x2000), out_dtype,
                                      G, R, C, ctypes.byref(p), ctypes.c_void_p(ws_ptr), ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(steps=0), 1),
    (dict(steps=65), 1),
    (dict(coeffs=[1.0, 2.0]), 1),
    (dict(coeffs=[1.0, 2.0, float("nan")]), 1),
    (dict(mode=7), 1),
    (dict(restart_after=-1), 1),
    (dict(safety=0.0), 1),
    (dict(safety=float("inf")), 1),
    (dict(eps=-1.0), 1),
    (dict(compute_dtype=9), 2),
    (dict(in_dtype=3), 2),
    (dict(out_dtype=-1), 2),
    (dict(G=-1), 3),
    (dict(R=70000), 3),
    (dict(ws_bytes=16), 4),
    (dict(ws_ptr=(1 << 20) + 8), 4),
])
def test_validation_before_launch(kw, code):
    assert _call(**kw) == code


def test_sym_updates_must_be_0_or_1():
    p, keep = nsg.make_params()
    p.sym_updates = 2
    out = ctypes.c_size_t(0)
    assert nsg.lib().ns_workspace_size(1, 64, 128, ctypes.byref(p), ctypes.byref(out)) == 1
    p.sym_updates = 1
    assert nsg.lib().ns_workspace_size(1, 64, 128, ctypes.byref(p), ctypes.byref(out)) == 0


def test_empty_bucket_is_a_no_op():
    assert _call(G=0) == 0
    assert _call(R=0) == 0
    assert _call(C=0) == 0
    assert nsg.workspace_size(0, 10, 10) == 0


def test_null_pointers_rejected():
    p, keep = nsg.make_params()
    L = nsg.lib()
    assert L.ns_orthogonalize(None, 0, ctypes.c_void_p(0x2000), 0, 1, 8, 8, ctypes.byref(p),
                              ctypes.c_void_p(1 << 20), 1 << 30, None, None) == 1
    assert L.ns_orthogonalize(ctypes.c_void_p(0x1000), 0, ctypes.c_void_p(0x2000), 0, 1, 8, 8, None,
                              ctypes.c_void_p(1 << 20), 1 << 30, None, None) == 1


@pytest.mark.parametrize("R,C", [(128, 512), (768, 3072), (11008, 4096), (2048, 512), (300, 1000), (1000, 300)])
def test_credited_flops_match_gram_formula(R, C):
    n, m = min(R, C), max(R, C)
    cr, ex = nsg.flops(R, C)
    assert cr == pytest.approx(oracle.flops_gram_stable(n, m, 5), rel=1e-12)
    assert ex >= 0.5 * cr


@pytest.mark.parametrize("R,C", [(4096, 4096), (333, 333), (128, 512)])
def test_credited_flops_standard(R, C):
    n, m = min(R, C), max(R, C)
    cr, _ = nsg.flops(R, C, mode="standard")
    assert cr == pytest.approx(oracle.flops_standard(n, m, 5), rel=1e-12)


def test_square_gram_falls_back_to_standard():
    labels = [e["label"] for e in nsg.plan(4096, 4096, mode="gram")]
    assert "R0=XXt" not in labels and labels.count("A=XXt") == 5
    cr, _ = nsg.flops(4096, 4096, mode="gram")
    assert cr == pytest.approx(oracle.flops_standard(4096, 4096, 5))


def test_gram_plan_structure():
    """Alg. 3: R0, then per step Z (+Q for a fresh Q), Q update, RZ and R; the
    restart (X=QX, R=XX^T) at the top of step 3; R_2 and R_5 skipped; 18 GEMMs."""
    P = nsg.plan(11008, 4096, in_dtype="bf16")
    labels = [e["label"] for e in P]
    gemms = [e for e in P if e["kernel"].startswith("gemm")]
    assert len(gemms) == 18
    assert labels[:3] == ["norm_reduce", "scale_cast_T", "R0=XXt"]
    steps = {}
    for e in P:
        steps.setdefault(e["step"], []).append(e["label"])
    assert steps[1] == ["Z (+Q=Z+aI)", "RZ=RZ+aR", "R=Z.RZ+aRZ"]
    assert steps[2] == ["Z=bR+cR2", "Q=QZ+aQ"]
    # tall input: only X^T is kept, so the restart forms X^T = X^T Q^T
    assert steps[3] == ["Xt=XtQt", "R=XXt", "Z (+Q=Z+aI)", "RZ=RZ+aR", "R=Z.RZ+aRZ"]
    assert steps[5] == ["Z=bR+cR2", "Q=QZ+aQ"]
    assert steps[6] == ["Yt=XtQt"]  # tall input: output written as Y^T, i.e. R x C
    assert [e["label"] for e in nsg.plan(768, 3072)][-1] == "Y=QX"
    # without a restart: Alg. 2 (with the implicit a I form)
    labels0 = [e["label"] for e in nsg.plan(768, 3072, restart_after=0)]
    assert "X=QX" not in labels0 and labels0.count("Q=QZ+aQ") == 4


def test_executed_flops_sum_of_plan():
    P = nsg.plan(768, 3072)
    _, ex = nsg.flops(768, 3072)
    assert ex == pytest.approx(sum(e["flops"] for e in P))


def test_workspace_scales_with_bucket():
    a = nsg.workspace_size(1, 11008, 4096)
    b = nsg.workspace_size(32, 11008, 4096)
    assert 31 * a <= b <= 32 * a + 32 * 256
    assert a % 256 == 0 and b % 256 == 0


def test_sym_updates_plan():
    """Q Z + a Q and R Z + a R on the symmetric kernel: same launches and
    credited FLOPs, lower-triangle tiles only, no transposed RZ buffer."""
    base = nsg.plan(11008, 4096, sym_updates=False)
    symp = nsg.plan(11008, 4096)
    assert [e["label"] for e in base] == [e["label"] for e in symp]
    for e0, e1 in zip(base, symp):
        if e0["label"] in ("Q=QZ+aQ", "RZ=RZ+aR"):
            assert e0["kernel"] == "gemm_nt" and e1["kernel"] == "gemm_nt_sym"
            assert e1["flops"] == pytest.approx(e0["flops"] * 136 / 256)  # 16 x 16 tiles -> 136
        else:
            assert e0["kernel"] == e1["kernel"] and e0["flops"] == e1["flops"]
    cr0, ex0 = nsg.flops(11008, 4096, sym_updates=False)
    cr1, ex1 = nsg.flops(11008, 4096)
    assert cr0 == cr1 and ex1 < ex0
    assert ex1 == pytest.approx(sum(e["flops"] for e in symp))
    # RZ^T is not kept: one n x n buffer less per matrix
    w0 = nsg.workspace_size(1, 11008, 4096, sym_updates=False)
    w1 = nsg.workspace_size(1, 11008, 4096)
    assert w0 - w1 >= 4096 * 4096 * 2
    # standard mode ignores it
    assert [e["kernel"] for e in nsg.plan(4096, 4096)] == [e["kernel"] for e in nsg.plan(4096, 4096, sym_updates=False)]


def test_restart_mask_validation_and_plan():
    p, keep = nsg.make_params(steps=6)
    out = ctypes.c_size_t(0)
    for mask, code in ((1, 1), (1 << 6, 1), (1 << 5, 0), (0b101010, 0)):
        p.restart_mask = mask
        assert nsg.lib().ns_workspace_size(1, 64, 128, ctypes.byref(p), ctypes.byref(out)) == code, mask
    with pytest.raises(ValueError):
        nsg.make_params(restarts=[0])
    P = nsg.plan(768, 3072, steps=10, restarts=[3, 6, 9])
    steps = {}
    for e in P:
        steps.setdefault(e["step"], []).append(e["label"])
    for t in (3, 6, 9):
        assert steps[t][:2] == ["X=QX", "R=XXt"] and steps[t][2] == "Z (+Q=Z+aI)"
        assert "R=Z.RZ+aRZ" not in steps[t - 1]  # R before a restart is not needed
    assert sum(lbl == "X=QX" for lbl in (e["label"] for e in P)) == 3


@pytest.mark.parametrize("T,restarts", [(5, [3]), (8, [3, 5]), (10, [2, 4, 6, 8])])
def test_credited_flops_several_restarts(T, restarts):
    """(4T + 3 alpha - 3) n^3 plus 3 (alpha - 1) n^3 per restart (Dion3 paper,
    Section 4.2: each restart costs 3 (alpha - 1) n^3)."""
    n, m = 768, 3072
    cr, _ = nsg.flops(n, m, steps=T, restarts=restarts)
    a = m / n
    assert cr == pytest.approx((4 * T + 3 * a - 3 + 3 * len(restarts) * (a - 1)) * n ** 3)


def test_select_validation_and_workspace():
    p, keep = nsg.make_params()
    out = ctypes.c_size_t(0)
    L = nsg.lib()
    # k out of range, bad dim
    assert L.ns_select_workspace_size(2, 64, 128, 0, 0, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 1
    assert L.ns_select_workspace_size(2, 64, 128, 65, 0, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 1
    assert L.ns_select_workspace_size(2, 64, 128, 10, 3, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 1
    assert L.ns_select_workspace_size(2, 64, 128, 10, 0, 7, 0, ctypes.byref(p), ctypes.byref(out)) == 2
    assert L.ns_select_workspace_size(2, 64, 128, 10, 0, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 0
    rows = out.value
    # smaller dimension of 64 x 128 is the rows: same as dim 0
    assert L.ns_select_workspace_size(2, 64, 128, 10, -1, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 0
    assert out.value == rows
    # columns of 256 x 100: k <= 100
    assert L.ns_select_workspace_size(1, 256, 100, 101, -1, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 1
    assert L.ns_select_workspace_size(1, 256, 100, 25, -1, 0, 0, ctypes.byref(p), ctypes.byref(out)) == 0
    # the inner workspace is included: at least ns_workspace_size of the submatrix
    inner = nsg.workspace_size(2, 10, 128)
    assert rows >= inner
    assert L.nsg_topk(None, 1, 10, 11, None, None, None) == 1
    assert nsg.select_count(4096, 0.25) == 1024 and nsg.select_count(10, 0.25) == 3
    assert nsg.select_count(4096, 0.25) == oracle.n_selected(4096, 0.25)


def test_select_count_rule_matches_the_oracle():
    """The library's k = ceil(f n) and default dimension (Dion3 paper,
    Section 6) against the selection oracle, over many shapes and fractions."""
    import itertools
    for (R, C), f in itertools.product([(4096, 11008), (11008, 4096), (100, 100), (1, 7), (7, 1), (333, 17)],
                                      [1e-3, 0.1, 0.25, 1 / 3, 0.5, 0.999, 1.0]):
        d, k = nsg.select_plan(R, C, f)
        assert d == oracle.select_dim(R, C), (R, C)
        n = R if d == 0 else C
        assert k == oracle.n_selected(n, f), (R, C, f)
        for dim in (0, 1):
            d2, k2 = nsg.select_plan(R, C, f, dim)
            assert d2 == dim and k2 == oracle.n_selected(R if dim == 0 else C, f)
    for bad in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(ValueError):
            nsg.select_plan(10, 20, bad)
    with pytest.raises(ValueError):
        nsg.select_plan(10, 20, 0.5, 2)
    assert nsg.select_plan(0, 20, 0.5, 0) == (0, 0)


# ---- Python-side buffer validation: every check runs before any launch ----

def test_out_shape_rules():
    """A caller's out must be exactly [G, R, C], or [R, C] for a single 2-D
    matrix: an [R, C] out for a bucket of G > 1 would be written G times over
    its end by the library."""
    import torch
    dev = torch.device("cpu")
    ok = torch.empty(3, 8, 16)
    nsg.check_out(ok, 3, 8, 16, False, dev)
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(8, 16), 3, 8, 16, False, dev)   # the overrun the rule exists for
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(8, 16), 1, 8, 16, False, dev)   # a 3-D input wants a 3-D out
    nsg.check_out(torch.empty(8, 16), 1, 8, 16, True, dev)         # 2-D input, 2-D out
    nsg.check_out(torch.empty(1, 8, 16), 1, 8, 16, True, dev)
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(2, 8, 16), 1, 8, 16, True, dev)
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(3, 16, 8), 3, 8, 16, False, dev)
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(3, 8, 32)[:, :, :16], 3, 8, 16, False, dev)  # not contiguous
    with pytest.raises(ValueError):
        nsg.check_out(torch.empty(3, 8, 16, dtype=torch.int32), 3, 8, 16, False, dev)
    with pytest.raises(ValueError):
        nsg.check_out(ok, 3, 8, 16, False, torch.device("meta"))  # another device


def test_status_and_workspace_rules():
    import torch
    dev = torch.device("cpu")
    nsg.check_status(None, 4, dev)
    nsg.check_status(torch.zeros(4, dtype=torch.int32), 4, dev)
    nsg.check_status(torch.zeros(9, dtype=torch.int32), 4, dev)
    for bad in (torch.zeros(3, dtype=torch.int32), torch.zeros(4, dtype=torch.int64),
                torch.zeros(8, dtype=torch.int32)[::2]):
        with pytest.raises(ValueError):
            nsg.check_status(bad, 4, dev)
    with pytest.raises(ValueError):
        nsg.check_status(torch.zeros(4, dtype=torch.int32), 4, torch.device("meta"))
    nsg.check_workspace(torch.empty(64, dtype=torch.uint8), dev)
    with pytest.raises(ValueError):
        nsg.check_workspace(torch.empty(64, dtype=torch.uint8), torch.device("meta"))
    assert nsg.nbytes(torch.empty(10, dtype=torch.float32)) == 40


def test_noalloc_rejects_before_any_gpu_call():
    """ns_orthogonalize_noalloc checks its arguments and the bucket's workspace
    against its fixed scratch before it touches a device."""
    L = nsg.lib()
    p, keep = nsg.make_params()
    fake_in, fake_out = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    # the 7B bucket needs ~17 GB of workspace: more than the fixed scratch
    assert nsg.workspace_size(32, 11008, 4096) > nsg.NOALLOC_MAX_BYTES
    assert L.ns_orthogonalize_noalloc(fake_in, 1, fake_out, 1, 32, 11008, 4096, ctypes.byref(p), None, None) == 6
    assert L.ns_status_string(6).decode() == nsg.STATUS[6]
    # argument errors as for ns_orthogonalize
    bad, keep2 = nsg.make_params(steps=0)
    assert L.ns_orthogonalize_noalloc(fake_in, 0, fake_out, 0, 2, 64, 128, ctypes.byref(bad), None, None) == 1
    assert L.ns_orthogonalize_noalloc(fake_in, 9, fake_out, 0, 2, 64, 128, ctypes.byref(p), None, None) == 2
    assert L.ns_orthogonalize_noalloc(None, 0, fake_out, 0, 2, 64, 128, ctypes.byref(p), None, None) == 1
    assert L.ns_orthogonalize_noalloc(fake_in, 0, fake_out, 0, -1, 64, 128, ctypes.byref(p), None, None) == 3
    # an empty bucket is a no-op
    assert L.ns_orthogonalize_noalloc(None, 0, None, 0, 0, 64, 128, ctypes.byref(p), None, None) == 0
    assert "NSG_NOALLOC_MAX_BYTES (128u << 20)" in open(HEADER).read()


def test_single_layout_plan():
    """The 16-bit 256 x 256 path keeps X in one layout only (the input's own):
    a tall input's Gram products read X^T K-major, a wide input's Q X reads X
    K-major, and no transposed copy of X is stored; the fp32 path and n <= 128
    (128 x 128 kernel) keep both layouts and row-major operands only; n = 200
    takes the 256 x 256 path."""
    def km(P):
        return {e["label"]: (e["a_kmajor"], e["b_kmajor"]) for e in P if e["kernel"].startswith("gemm")}
    tall = km(nsg.plan(11008, 4096))
    assert tall["R0=XXt"] == (True, True) and tall["R=XXt"] == (True, True)
    assert tall["Xt=XtQt"] == (False, False) and tall["Yt=XtQt"] == (False, False)
    assert all(v == (False, False) for k, v in tall.items() if k not in ("R0=XXt", "R=XXt"))
    wide = km(nsg.plan(768, 3072))
    assert wide["X=QX"] == (False, True) and wide["Y=QX"] == (False, True)
    assert wide["R0=XXt"] == (False, False) and wide["R=XXt"] == (False, False)
    sq = nsg.plan(4096, 4096)
    assert all(e["b_kmajor"] and not e["a_kmajor"] for e in sq if e["label"] in ("X=aX+BX", "Y=aX+BX"))
    tall_std = km(nsg.plan(4096, 1024, mode="standard"))
    assert tall_std["A=XXt"] == (True, True) and tall_std["Xt=aXt+XtB"] == (False, False)
    for P in (nsg.plan(11008, 4096, compute_dtype="f32"), nsg.plan(100, 1000), nsg.plan(1000, 128)):
        assert not any(e["a_kmajor"] or e["b_kmajor"] for e in P)
    assert km(nsg.plan(200, 1000))["X=QX"] == (False, True)
    # one copy of X (and of X after the restart) instead of two
    n, m, es = 4096, 11008, 2
    x_bytes = m * (n + 64) * es
    assert nsg.workspace_size(1, 11008, 4096) < 2 * x_bytes + 6 * n * (n + 64) * es
    assert nsg.workspace_size(1, 11008, 4096, compute_dtype="f32") > 4 * m * n * 4


def test_in_place_plan():
    """A 16-bit input in the compute dtype with both sides multiples of 256 is
    read in place: the scale pass only finds the scales and writes no copy
    (no bytes), the launches and the other entries are unchanged, and so is
    the workspace.  A ragged side, fp32 compute and the 128 x 128 path
    (n <= 128) keep the copy."""
    def desc(P):
        return [(e["label"], e["kernel"], e["flops"], e["a_kmajor"], e["b_kmajor"]) for e in P]
    for R, C, kw in ((2048, 512, {}), (768, 3072, {}), (4096, 4096, {}), (2048, 512, dict(mode="standard")),
                     (512, 1024, dict(steps=8, restarts=[3, 5]))):
        direct = nsg.plan(R, C, in_dtype="f16", **kw)
        copy = nsg.plan(R, C, in_dtype="f32", **kw)
        assert direct[1]["label"] == "scales" and direct[1]["bytes"] == 0
        assert copy[1]["label"] == "scale_cast_T"
        assert copy[1]["bytes"] == R * C * 4 + R * C * 2
        assert desc(direct)[2:] == desc(copy)[2:]
        assert [e["bytes"] for e in direct[2:]] == [e["bytes"] for e in copy[2:]]
        assert all(e["source"] == 0 for e in direct + copy)
    # the norm reads the input in its own dtype
    assert nsg.plan(2048, 512, in_dtype="f32")[0]["bytes"] == 2048 * 512 * 4
    for R, C, kw in ((2000, 512, {}), (768, 3000, {}), (2048, 512, dict(compute_dtype="f32")), (2048, 128, {}),
                     (128, 1024, {})):
        assert nsg.plan(R, C, in_dtype=kw.get("compute_dtype", "f16"), **kw)[1]["label"] == "scale_cast_T"
        assert nsg.plan(R, C, in_dtype="bf16", **kw)[1]["label"] == "scale_cast_T"
    # n = 256 runs on the 256 x 256 kernel and is read in place as well
    for R, C in ((2048, 256), (256, 1024)):
        assert nsg.plan(R, C, in_dtype="f16")[1]["label"] == "scales"
    with pytest.raises(nsg.NSGError):
        nsg.plan(2048, 512, in_dtype=7)


def test_bf16_input_plan():
    """A bf16 input under fp16 compute, both sides multiples of 256,
    256 <= n < 2048: the scale pass writes no copy, the first X X^T (R0, or
    the standard step's A) multiplies the raw bf16 input (source 3) and the
    general products that read X0 convert it (source 1 for A, 2 for the
    K-major B); everything else is the plan of an fp16 input.  n >= 2048,
    ragged sides, n <= 128 and bf16 compute keep the copy."""
    def desc(P):
        return [(e["label"], e["kernel"], e["flops"], e["a_kmajor"], e["b_kmajor"], e["bytes"]) for e in P]
    for R, C, kw, x0_readers in (
            (2048, 512, {}, {"R0=XXt": 3, "Xt=XtQt": 1}),
            (768, 3072, {}, {"R0=XXt": 3, "X=QX": 2}),
            (4096, 1536, {}, {"R0=XXt": 3, "Xt=XtQt": 1}),
            (2048, 512, dict(restart_after=0), {"R0=XXt": 3, "Yt=XtQt": 1}),
            (512, 2048, dict(steps=1), {"R0=XXt": 3, "Y=QX": 2}),
            (512, 1024, dict(steps=8, restarts=[3, 5]), {"R0=XXt": 3, "X=QX": 2}),
            (768, 768, {}, {"A=XXt": 3, "X=aX+BX": 2}),
            (2048, 512, dict(mode="standard"), {"A=XXt": 3, "Xt=aXt+XtB": 1}),
            (512, 1536, dict(mode="standard"), {"A=XXt": 3, "X=aX+BX": 2}),
            (1536, 1536, dict(steps=1), {"A=XXt": 3, "Y=aX+BX": 2}),
            (256, 1024, {}, {"R0=XXt": 3, "X=QX": 2})):
        P = nsg.plan(R, C, in_dtype="bf16", **kw)
        assert P[1]["label"] == "scales" and P[1]["bytes"] == 0
        sources = [(e["label"], e["source"]) for e in P if e["source"]]
        # exactly the first launch of each X0 reader (a later restart reads X1)
        assert dict(sources) == x0_readers and len(sources) == len(x0_readers), sources
        assert desc(P)[2:] == desc(nsg.plan(R, C, in_dtype="f16", **kw))[2:]
    for R, C, kw in ((4096, 4096, {}), (2048, 2048, {}), (2048, 512, dict(compute_dtype="bf16")),
                     (2000, 512, {}), (128, 1024, {}), (11008, 4096, {}), (2048, 8192, {})):
        P = nsg.plan(R, C, in_dtype="bf16", **kw)
        assert all(e["source"] == 0 for e in P), (R, C, kw)
        assert P[1]["label"] == ("scales" if kw.get("compute_dtype") == "bf16" else "scale_cast_T")
