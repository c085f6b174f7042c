"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars per matrix (tests/parity_metrics.py defines the measures):
  * relative Frobenius error <= 3e-2 and cosine >= 0.97 for the fp16/bf16
    paths, relative error <= 1e-4 for the fp32 debug path (the pages' bars);
  * on the full-size buckets also a worst 256 x 256 block error and a worst
    single-element error, both against the matrix's RMS entry: a wrong tile,
    or a corner of one, fails these while it barely moves the whole-matrix
    norm.  Their bars are fixed multiples of the errors these kernels show on
    the same seeded inputs (recorded with the bars below);
  * grouped and single-matrix outputs bitwise identical; repeated calls
    bitwise identical.
"""
import json
import os

import numpy as np
import pytest
import torch

import newton_schulz_gram_amd as nsg
import oracle
import synth
from parity_metrics import bucket_errors, summary
from synth import COEFFS_MUON, WORKLOADS
from synth.workloads import conditioning_class_of, custom

pytestmark = pytest.mark.gpu

HALF_REL, HALF_COS, F32_REL = 3e-2, 0.97, 1e-4

# Localized bars: worst 256 x 256 block RMS error and worst element error,
# both divided by the matrix's RMS entry, per conditioning class (the
# full-size buckets are Gaussian).  Each bar is about three times the worst
# value these kernels show on the seeded inputs (default and stress setups,
# symmetric and general updates): Gaussian-like classes and the 7B, square and
# MoE buckets reach 2.1e-3 (block) and 0.026 (element); ill-conditioned 0.016
# and 0.11; low-rank 0.030 and 0.27; heavy-tailed 0.0024 and 0.27 (its large
# entries carry proportionally large errors).  A wrong tile scores ~1 on the
# block measure, a wrong sixteenth of one ~0.25.
BLOCK_BAR = {"gaussian": 1e-2, "ill_conditioned": 5e-2, "low_rank": 9e-2, "heavy_tailed": 1e-2,
             "scaled_up": 1e-2, "scaled_down": 1e-2, "near_orthogonal": 1e-2}
ELEM_BAR = {"gaussian": 0.1, "ill_conditioned": 0.35, "low_rank": 0.8, "heavy_tailed": 0.8,
            "scaled_up": 0.1, "scaled_down": 0.1, "near_orthogonal": 0.1}


def metrics(out, ref):
    """Per-matrix (relative Frobenius error, cosine) of out vs the fp64 ref."""
    o = out.double().cpu().numpy().reshape(out.shape[0], -1)
    r = np.asarray(ref, dtype=np.float64).reshape(o.shape[0], -1)
    d = np.linalg.norm(o - r, axis=1)
    rn = np.linalg.norm(r, axis=1)
    on = np.linalg.norm(o, axis=1)
    rel = d / np.maximum(rn, 1e-300)
    cos = np.sum(o * r, axis=1) / np.maximum(on * rn, 1e-300)
    return rel, cos


def run(x, **kw):
    y = nsg.orthogonalize(x.cuda(), **kw)
    torch.cuda.synchronize()
    return y


def oracle_of(x, mode="gram", steps=5, coeffs=COEFFS_MUON, restart_after=2, safety=1.05):
    return oracle.orthogonalize(x.double().numpy(), steps, coeffs, mode, restart_after, safety)


def check(out, ref, compute, label=""):
    rel, cos = metrics(out, ref)
    if compute == "f32":
        assert rel.max() <= F32_REL, (label, rel.max())
    else:
        assert rel.max() <= HALF_REL, (label, rel.max(), int(rel.argmax()))
        assert cos.min() >= HALF_COS, (label, cos.min())
    return rel, cos


def record(label, stats):
    """Print one line of measured errors, and append it to
    parity_errors.jsonl in the folder NSG_RECORD_DIR names, if it is set."""
    line = json.dumps({"case": label, **{k: (round(v, 7) if isinstance(v, float) else v)
                                         for k, v in stats.items()}})
    print(line, flush=True)
    d = os.environ.get("NSG_RECORD_DIR")
    if d and os.path.isdir(d):
        with open(os.path.join(d, "parity_errors.jsonl"), "a") as fh:
            fh.write(line + "\n")


def check_local(out, ref, label, cls="gaussian"):
    """Every bar on every matrix: rel / cos, worst block, worst element."""
    errs = bucket_errors(out, ref)
    s = summary(errs)
    record(label, s)
    assert s["rel_max"] <= HALF_REL, (label, s)
    assert s["cos_min"] >= HALF_COS, (label, s)
    assert s["block_rel_max"] <= BLOCK_BAR[cls], (label, s)
    assert s["elem_max"] <= ELEM_BAR[cls], (label, s)
    return errs


# ---------------------------------------------------------------------------
# single fp32 128x512 matrix, both modes, fp32 and fp16 compute
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["gram", "standard"])
@pytest.mark.parametrize("compute", ["f32", "f16", "bf16"])
def test_single_128x512(mode, compute):
    w = WORKLOADS["single_1x128x512_f32"]
    x = synth.make(w)
    ref = oracle_of(x, mode=mode, safety=1.0)
    out = run(x, mode=mode, safety=1.0, compute_dtype=compute)
    assert out.dtype == torch.float32
    check(out, ref, compute, f"{mode}/{compute}")


# ---------------------------------------------------------------------------
# ragged and odd shapes, several tiles plus a tail
# ---------------------------------------------------------------------------

SHAPES = [(300, 1000), (1000, 300), (333, 333), (257, 513), (1, 50), (50, 1), (7, 9), (130, 4000),
          (384, 768)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_ragged_shapes_fp16(shape, mode):
    R, C = shape
    x = custom(3, R, C, "f16", "gaussian", seed=21)
    ref = oracle_of(x, mode=mode)
    out = run(x, mode=mode)
    assert out.shape == x.shape and out.dtype == torch.float16
    check(out, ref, "f16", f"{shape}/{mode}")


@pytest.mark.parametrize("shape", [(300, 1000), (1000, 300), (333, 333)])
@pytest.mark.parametrize("compute", ["f32", "bf16"])
def test_ragged_shapes_other_compute(shape, compute):
    R, C = shape
    x = custom(2, R, C, "f32", "gaussian", seed=22)
    ref = oracle_of(x)
    out = run(x, compute_dtype=compute)
    check(out, ref, compute, f"{shape}/{compute}")


@pytest.mark.parametrize("restart_after", [0, 1, 2, 3, 4, 5])
def test_every_restart_location(restart_after):
    x = custom(2, 256, 1024, "f16", "gaussian", seed=23)
    ref = oracle_of(x, restart_after=restart_after)
    out = run(x, restart_after=restart_after)
    check(out, ref, "f16", f"restart {restart_after}")


def test_per_step_coefficients_and_steps():
    coeffs = [3.4445, -4.7750, 2.0315, 15 / 8, -10 / 8, 3 / 8, 2.0, -1.5, 0.5]
    x = custom(2, 200, 600, "f16", "gaussian", seed=24)
    for mode in ("gram", "standard"):
        ref = oracle_of(x, mode=mode, steps=3, coeffs=coeffs, restart_after=1)
        out = run(x, mode=mode, steps=3, coeffs=coeffs, restart_after=1, compute_dtype="f32",
                  out_dtype=torch.float32)
        check(out, ref, "f32", mode)


# ---------------------------------------------------------------------------
# GPT-2-small MLP bucket: 42 x 768x3072, seven conditionings
# ---------------------------------------------------------------------------

def per_class(w, out, ref, label):
    """Bars per conditioning class (every matrix of the class)."""
    o = out.double().cpu().numpy()
    by = {}
    for g in range(w.G):
        by.setdefault(conditioning_class_of(w.G, g), []).append(g)
    worst = {}
    for cls, idx in by.items():
        worst[cls] = check_local(o[idx], ref[idx], f"{label}/{cls}", cls)
    return {c: max(e["rel"] for e in v) for c, v in worst.items()}


def test_gpt2s_bucket_all_conditionings():
    w = WORKLOADS["gpt2s_mlp_42x768x3072_f16"]
    x = synth.make(w)
    ref = oracle_of(x, safety=w.safety)
    out = run(x, safety=w.safety)
    worst = per_class(w, out, ref, "gpt2s")
    print("per-class max rel error:", {k: round(v, 5) for k, v in worst.items()})
    # grouped == single, bitwise
    for g in (0, 13, 41):
        one = run(x[g:g + 1], safety=w.safety)
        assert torch.equal(one[0], out[g])
    # repeated call, bitwise
    again = run(x, safety=w.safety)
    assert torch.equal(again, out)


def test_gpt2s_forced_symmetry_under_stress():
    """Forced symmetry under the pages' stress setup (Dion3 paper, App. B.2.3:
    restart after three steps instead of two, safety 1.02 instead of 1.05):
    symmetric updates (Q Z + a Q and R Z + a R computed as lower triangles and
    mirrored) against general updates, every conditioning class.  Both must
    stay finite with a clear status flag and within the bars, and the
    symmetric form may not be worse than the general one on any class by more
    than a quarter (plus 1e-3 of slack for rounding order)."""
    w = WORKLOADS["gpt2s_mlp_42x768x3072_f16"]
    x = synth.make(w)
    ref = oracle_of(x, restart_after=3, safety=1.02)
    xc = x.cuda()
    res = {}
    for sym in (True, False):
        st = torch.full((w.G,), 7, dtype=torch.int32, device="cuda")
        out = nsg.orthogonalize(xc, restart_after=3, safety=1.02, sym_updates=sym, status=st)
        torch.cuda.synchronize()
        assert st.sum().item() == 0, st.tolist()
        assert bool(torch.isfinite(out.float()).all())
        res[sym] = per_class(w, out, ref, f"gpt2s_stress_r3_s1.02/{'sym' if sym else 'gen'}")
    print("stress per-class max rel error (sym, gen):",
          {c: (round(res[True][c], 5), round(res[False][c], 5)) for c in res[True]})
    for c in res[True]:
        assert res[True][c] <= 1.25 * res[False][c] + 1e-3, (c, res[True][c], res[False][c])


# ---------------------------------------------------------------------------
# MoE bucket: 512 x 2048x512 (transposed to 512 x 2048)
# ---------------------------------------------------------------------------

def test_moe_bucket_sampled():
    w = WORKLOADS["moe_512x2048x512_f16"]
    x = synth.make(w)
    out = run(x, safety=w.safety)
    idx = sorted(set(list(range(0, 512, 16)) + [1, 77, 255, 300, 511]))
    ref = oracle_of(x[idx], safety=w.safety)
    check_local(out[idx], ref, f"moe x{len(idx)}")
    for g in (0, 300):
        one = run(x[g:g + 1], safety=w.safety)
        assert torch.equal(one[0], out[g])


# ---------------------------------------------------------------------------
# Full-size buckets, sampled against the oracle (four matrices each, every
# element and every 256 x 256 block checked)
# ---------------------------------------------------------------------------

def test_llama7b_bucket_sampled():
    w = WORKLOADS["llama7b_mlp_32x11008x4096_bf16"]
    x = synth.make(w)
    out = run(x, safety=w.safety)
    assert out.dtype == torch.bfloat16 and out.shape == (32, 11008, 4096)
    idx = [0, 11, 22, 31]
    o = out[idx].cpu()
    one = run(x[5:6], safety=w.safety)
    assert torch.equal(one[0], out[5])
    del out, one
    ref = oracle_of(x[idx], safety=w.safety)
    check_local(o, ref, "llama7b x4")


def test_square_bucket_standard_fallback_sampled():
    w = WORKLOADS["square_32x4096x4096_f16"]
    x = synth.make(w)
    out = run(x, safety=w.safety)
    idx = [0, 10, 21, 31]
    o = out[idx].cpu()
    one = run(x[10:11], safety=w.safety)
    assert torch.equal(one[0], out[10])
    del out, one
    ref = oracle_of(x[idx], safety=w.safety)
    check_local(o, ref, "square x4")


# ---------------------------------------------------------------------------
# Edge cases and API behaviour
# ---------------------------------------------------------------------------

def test_zero_matrix_and_status():
    x = torch.zeros(2, 64, 256, dtype=torch.float16)
    x[1] = torch.from_numpy(np.random.default_rng(0).standard_normal((64, 256))).half()
    st = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    out = nsg.orthogonalize(x.cuda(), status=st)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    assert st.tolist() == [0, 0]


def test_non_finite_input_sets_status():
    x = torch.randn(3, 64, 256).half()
    x[1, 3, 5] = float("inf")
    st = torch.zeros(3, dtype=torch.int32, device="cuda")
    out = nsg.orthogonalize(x.cuda(), status=st)
    torch.cuda.synchronize()
    assert st.tolist() == [0, 1, 0]
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[2]).all()


def test_naive_gram_blow_up_raises_status():
    """Gram NS without a restart (Dion3 paper, Algorithm 2) in fp16 on a rank-16
    matrix, run for T = 10 steps: the spurious eigenvalues of the iterated Gram
    matrix grow until the output is non-finite (the pages' App. B failure
    mode), and the status flag reports it without a host synchronisation.  The
    recommended setup (T = 5, restart before step 3) on the same matrix stays
    finite and clear."""
    rng = np.random.default_rng(5)
    x = torch.from_numpy((rng.standard_normal((512, 16)) @ rng.standard_normal((16, 2048))).astype(np.float32))
    x = x[None].half().cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = nsg.orthogonalize(x, steps=10, mode="gram", restart_after=0, compute_dtype=torch.float16, status=st)
    torch.cuda.synchronize()
    assert st.item() == 1 and not bool(torch.isfinite(y.float()).all())
    st[0] = 7
    y = nsg.orthogonalize(x, steps=5, mode="gram", restart_after=2, compute_dtype=torch.float16, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0 and bool(torch.isfinite(y.float()).all())


def test_in_place_and_output_dtype():
    x = custom(2, 200, 500, "f16", "gaussian", seed=31)
    ref = oracle_of(x)
    xc = x.cuda()
    y32 = nsg.orthogonalize(xc, out_dtype=torch.float32)
    y = nsg.orthogonalize(xc, out=xc)  # in place
    torch.cuda.synchronize()
    assert y.data_ptr() == xc.data_ptr()
    check(y, ref, "f16")
    check(y32, ref, "f16")
    assert y32.dtype == torch.float32


def test_empty_bucket():
    x = torch.zeros(0, 16, 32, dtype=torch.float16, device="cuda")
    assert nsg.orthogonalize(x).shape == (0, 16, 32)


def test_single_matrix_2d_input():
    x = custom(1, 100, 300, "bf16", "gaussian", seed=32)
    out = nsg.orthogonalize(x[0].cuda())
    torch.cuda.synchronize()
    assert out.shape == (100, 300) and out.dtype == torch.bfloat16
    check(out.unsqueeze(0), oracle_of(x), "f16")


# ---------------------------------------------------------------------------
# General Q Z + a Q and R Z + a R (sym_updates=False; the default runs them
# on the symmetric kernel): every conditioning class, the restart locations
# and the full-size buckets
# ---------------------------------------------------------------------------

def test_general_updates_gpt2s_all_conditionings():
    w = WORKLOADS["gpt2s_mlp_42x768x3072_f16"]
    x = synth.make(w)
    ref = oracle_of(x, safety=w.safety)
    out = run(x, safety=w.safety, sym_updates=False)
    rel, cos = metrics(out, ref)
    worst = {}
    for g in range(w.G):
        c = conditioning_class_of(w.G, g)
        worst[c] = max(worst.get(c, 0.0), float(rel[g]))
    print("general updates per-class max rel error:", {k: round(v, 5) for k, v in worst.items()})
    assert rel.max() <= HALF_REL, worst
    assert cos.min() >= HALF_COS
    for g in (0, 20, 41):
        one = run(x[g:g + 1], safety=w.safety, sym_updates=False)
        assert torch.equal(one[0], out[g])


@pytest.mark.parametrize("compute", ["f32", "f16", "bf16"])
def test_general_updates_single_128x512(compute):
    x = synth.make(WORKLOADS["single_1x128x512_f32"])
    ref = oracle_of(x, safety=1.0)
    out = run(x, safety=1.0, compute_dtype=compute, sym_updates=False, out_dtype=torch.float32)
    check(out, ref, compute, f"general updates {compute}")


@pytest.mark.parametrize("restart_after", [0, 1, 3, 4])
def test_general_updates_restart_locations(restart_after):
    x = custom(2, 256, 1024, "f16", "gaussian", seed=23)
    ref = oracle_of(x, restart_after=restart_after)
    out = run(x, restart_after=restart_after, sym_updates=False)
    check(out, ref, "f16", f"general updates restart {restart_after}")


def test_general_updates_moe_and_llama7b_sampled():
    w = WORKLOADS["moe_512x2048x512_f16"]
    x = synth.make(w)
    out = run(x, safety=w.safety, sym_updates=False)
    idx = [0, 255, 511]
    check(out[idx], oracle_of(x[idx], safety=w.safety), "f16", "moe general updates")
    del x, out
    w = WORKLOADS["llama7b_mlp_32x11008x4096_bf16"]
    x = synth.make(w)
    out = run(x, safety=w.safety, sym_updates=False)
    rel, cos = check(out[:1], oracle_of(x[:1], safety=w.safety), "f16", "7b general updates")
    print("7b general updates matrix 0: rel %.3e cos %.6f" % (rel[0], cos[0]))
    one = run(x[7:8], safety=w.safety, sym_updates=False)
    assert torch.equal(one[0], out[7])


# ---------------------------------------------------------------------------
# Several restarts (restart_mask) and per-step coefficient schedules
# ---------------------------------------------------------------------------

MIXED10 = [3.4445, -4.7750, 2.0315] * 5 + [15 / 8, -10 / 8, 3 / 8] * 5


@pytest.mark.parametrize("steps,restarts", [(8, [3, 5]), (10, [2, 4, 6, 8]), (10, [5]), (6, [2, 3, 4, 5, 6])])
def test_several_restarts(steps, restarts):
    coeffs = (MIXED10[:15] + MIXED10[-3 * (steps - 5):]) if steps > 5 else MIXED10[:3 * steps]
    x = custom(3, 256, 1024, "f16", "gaussian", seed=41)
    ref = oracle.orthogonalize(x.double().numpy(), steps, coeffs, "gram", 0, 1.05, restarts=restarts)
    out = run(x, steps=steps, coeffs=coeffs, restarts=restarts)
    check(out, ref, "f16", f"restarts {restarts}")
    out32 = run(x, steps=steps, coeffs=coeffs, restarts=restarts, compute_dtype="f32", out_dtype=torch.float32)
    check(out32, ref, "f32", f"restarts {restarts} fp32")


# ---------------------------------------------------------------------------
# A 16-bit input in the compute dtype, with both sides multiples of 256 and an
# output that does not overlap it, is read in place by the products (its
# per-matrix power of two 2^e rides in their fp32 scale) instead of through a
# scaled copy; out == in takes the copy.  Where the copy G 2^e is exact
# (e >= 0: scaling up never rounds) and no entry is an fp16 subnormal, the two
# routes give the same bits.  With subnormal entries they may differ in a few
# last bits: the f16 MFMA's sums over subnormal operands are not exactly
# invariant under a power-of-two scale (measured: about 1 output in 2000 of
# an all-subnormal operand moves by an ulp, with the same worst error against
# fp64 either way), so there both routes are held to the oracle instead.
# ---------------------------------------------------------------------------

IN_PLACE_CASES = [
    # G, R, C, params
    (4, 2048, 512, {}),                           # tall, Gram (MoE-like)
    (3, 768, 3072, {}),                           # wide, Gram (GPT-2-like)
    (2, 1024, 1024, {}),                          # square: standard NS
    (2, 2048, 512, dict(mode="standard")),        # tall, standard
    (2, 512, 1536, dict(mode="standard")),        # wide, standard
    (2, 2048, 512, dict(restart_after=0)),        # no restart: the output product reads the input
    (2, 512, 2048, dict(steps=1)),                # one step
    (2, 512, 1024, dict(steps=8, restarts=[3, 5], coeffs=MIXED10[:15] + MIXED10[-9:])),
]


def normal_range_gaussian(G, R, C, sigma, seed):
    """N(0, sigma^2) entries in fp16 with magnitudes below 2^-13 lifted to
    2^-13, so that no entry (nor its copy scaled up) is an fp16 subnormal."""
    x = custom(G, R, C, "f32", "gaussian", seed=seed) * sigma
    tiny = 2.0 ** -13
    x = torch.where(x.abs() < tiny, torch.where(x < 0, torch.full_like(x, -tiny), torch.full_like(x, tiny)), x)
    return x.half()


def both_routes(x, **kw):
    """(read in place, through the scaled copy) outputs of one input."""
    xc = x.cuda()
    y = nsg.orthogonalize(xc, **kw)
    x2 = xc.clone()
    y2 = nsg.orthogonalize(x2, out=x2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(xc, x.cuda())  # the input is never written
    return y, y2


@pytest.mark.parametrize("case", range(len(IN_PLACE_CASES)))
def test_input_read_in_place_matches_the_copy(case):
    G, R, C, kw = IN_PLACE_CASES[case]
    x = normal_range_gaussian(G, R, C, 1e-2, 60 + case)
    assert [e["label"] for e in nsg.plan(R, C, in_dtype="f16", **kw)][1] == "scales"
    y, y2 = both_routes(x, **kw)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), case
    if case in (0, 1, 2):
        check(y, oracle_of(x, mode=kw.get("mode", "gram")), "f16", f"in place {case}")


def test_input_read_in_place_bf16():
    """bf16 input with bf16 compute is read in place too (bf16 has fp32's
    exponent range, so the copy G 2^e is exact for N(0,1) entries): same bits
    as the copy route, tall and wide, and within the oracle's bars."""
    for case, (G, R, C) in enumerate(((3, 2048, 512), (2, 512, 1536))):
        x = custom(G, R, C, "bf16", "gaussian", seed=80 + case)
        kw = dict(compute_dtype="bf16")
        assert [e["label"] for e in nsg.plan(R, C, in_dtype="bf16", **kw)][1] == "scales"
        y, y2 = both_routes(x, **kw)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), case
        check(y, oracle_of(x), "bf16", f"in place bf16 {case}")


BF16_IN_PLACE_CASES = [
    # G, R, C, params
    (4, 2048, 512, {}),                           # tall: R0 of the raw input read K-major, X^T Q^T converts A
    (3, 768, 3072, {}),                           # wide: R0 row-major, Q X converts the K-major B
    (2, 2048, 512, dict(restart_after=0)),        # no restart: the output product converts
    (2, 512, 2048, dict(steps=1)),                # one step, wide
    (2, 512, 1024, dict(steps=8, restarts=[3, 5], coeffs=MIXED10[:15] + MIXED10[-9:])),
    (2, 1536, 512, dict(sym_updates=False)),      # general Q and RZ updates
    (2, 768, 768, {}),                            # square: standard NS, X = aX + BX converts B and Cin
    (2, 2048, 512, dict(mode="standard")),        # tall standard: X^T = aX^T + X^T B converts A and Cin
    (2, 512, 1536, dict(mode="standard", steps=1)),  # wide standard, one step: the output product converts
]


@pytest.mark.parametrize("case", range(len(BF16_IN_PLACE_CASES)))
def test_bf16_input_read_in_place_matches_the_copy(case):
    """A bf16 input under fp16 compute read in place: the first X X^T from
    the raw bf16 values on bf16 MFMAs, X0 converted on its way to LDS in the
    products that read it (and in the epilogue where it is the added term).
    On inputs whose X0 = G 2^e has no fp16-subnormal entry the bf16 values
    convert exactly, their products are the same in either MFMA, and the
    output has the copy route's bits."""
    G, R, C, kw = BF16_IN_PLACE_CASES[case]
    x = normal_range_gaussian(G, R, C, 1e-2, 90 + case).bfloat16()
    P = nsg.plan(R, C, in_dtype="bf16", **kw)
    assert P[1]["label"] == "scales" and {e["source"] for e in P} == {0, 3, 1 if R > C else 2}
    y, y2 = both_routes(x, **kw)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), case
    if case < 2 or case == 6:
        check(y, oracle_of(x.float(), mode=kw.get("mode", "gram"), safety=1.05), "f16", f"bf16 in place {case}")


@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_bf16_input_read_in_place_other_output_dtypes(out_dtype):
    """fp32 and fp16 outputs of a bf16 input read in place, against the copy
    route: a copy of the input 2 bytes past a 16-byte boundary is not read in
    place (the products need 16-byte rows), so it takes the scaled copy."""
    G, R, C = 3, 2048, 512
    x = normal_range_gaussian(G, R, C, 1e-2, 98).bfloat16().cuda()
    buf = torch.empty(G * R * C + 8, dtype=torch.bfloat16, device="cuda")
    xm = buf[1:1 + G * R * C].view(G, R, C)
    xm.copy_(x)
    assert x.data_ptr() % 16 == 0 and xm.data_ptr() % 16 == 2
    odt = {"f32": torch.float32, "f16": torch.float16}[out_dtype]
    y = nsg.orthogonalize(x, out_dtype=odt)
    y2 = nsg.orthogonalize(xm, out_dtype=odt)
    torch.cuda.synchronize()
    assert y.dtype == y2.dtype == odt
    assert torch.equal(y, y2)
    check(y, oracle_of(x.float().cpu()), "f16", f"bf16 in place, {out_dtype} output")


def test_bf16_input_read_in_place_degenerate_matrices():
    """A zero matrix (its exponent leaves the raw window: R0 reads the zero
    copy), one with a NaN and one with an infinity (read raw), next to a
    normal one: the status flags of both routes agree, the zero and the
    normal matrix keep the copy route's bits, the zero one's output is zero."""
    G, R, C = 4, 2048, 512
    x = normal_range_gaussian(G, R, C, 1e-2, 99).bfloat16().cuda()
    x[0].zero_()
    x[1, 5, 7] = float("nan")
    x[2, 100, 3] = float("inf")
    st = torch.full((G,), 7, dtype=torch.int32, device="cuda")
    st2 = torch.full((G,), 7, dtype=torch.int32, device="cuda")
    y = nsg.orthogonalize(x, status=st)
    x2 = x.clone()
    y2 = nsg.orthogonalize(x2, out=x2, status=st2)
    torch.cuda.synchronize()
    assert st.tolist() == st2.tolist() == [0, 1, 1, 0]
    for b in (0, 3):
        assert torch.equal(y[b].view(torch.int16), y2[b].view(torch.int16)), b
    assert not torch.any(y[0] != 0)


@pytest.mark.parametrize("R,C", [(2048, 512), (512, 1536)])
def test_bf16_input_outside_the_raw_range(R, C):
    """Matrices scaled by 2^-40 and 2^60 (|G|_F near 2^-30 and 2^70) fall
    outside the raw product's exponent window: the scale pass writes their
    bf16 copy G 2^e, R0 reads it, and every matrix of the bucket (those read
    raw too: scales 1 and 2^-20) keeps the copy route's bits."""
    x = normal_range_gaussian(4, R, C, 1e-2, 95).float()
    for b, k in enumerate((0, -40, 60, -20)):
        x[b] *= 2.0 ** k
    x = x.bfloat16()
    y, y2 = both_routes(x)
    for b in range(4):
        assert torch.equal(y[b].view(torch.int16), y2[b].view(torch.int16)), b
    check(y, oracle_of(x.float()), "f16", f"bf16 outside the raw range {R}x{C}")


@pytest.mark.parametrize("sigma", [1.0, 1e-3])
def test_bf16_input_read_in_place_gaussian(sigma):
    """Gaussian bf16 inputs (X0 holds fp16-subnormal entries, which the raw
    R0 keeps exact and the copy rounds): both routes meet the oracle bars and
    stay within 2e-3 of each other (measured 7e-4: once one rounding differs,
    the two runs part at the level of fp16's unit roundoff)."""
    x = (custom(3, 2048, 512, "f32", "gaussian", seed=97) * sigma).bfloat16()
    ref = oracle_of(x.float())
    y, y2 = both_routes(x)
    rel, _ = check(y, ref, "f16", f"bf16 in place, sigma {sigma}")
    rel2, _ = check(y2, ref, "f16", f"bf16 copy, sigma {sigma}")
    d = float((y.float() - y2.float()).norm() / y2.float().norm())
    record(f"bf16 in place vs copy, N(0,{sigma}^2)", {"in_place_rel_max": float(rel.max()),
                                                     "copy_rel_max": float(rel2.max()), "routes_rel_diff": d})
    assert d < 2e-3


@pytest.mark.parametrize("sigma,shape", [(1.0, (4, 2048, 512)), (1e-2, (4, 2048, 512)), (2e-5, (2, 2048, 512)),
                                         (1e-3, (2, 768, 3072))])
def test_input_read_in_place_with_subnormal_entries(sigma, shape):
    """Gaussian inputs with fp16-subnormal entries (2e-5: most of them; 1.0:
    the copy G 2^e, e < 0, rounds its smallest entries into subnormals):
    both routes meet the oracle bars."""
    x = (custom(*shape, "f32", "gaussian", seed=70) * sigma).half()
    ref = oracle_of(x)
    y, y2 = both_routes(x)
    rel, _ = check(y, ref, "f16", f"in place, sigma {sigma}")
    rel2, _ = check(y2, ref, "f16", f"copy, sigma {sigma}")
    d = (y.float() - y2.float()).norm() / y2.float().norm()
    record(f"in place vs copy, {shape} N(0,{sigma}^2)", {"in_place_rel_max": float(rel.max()),
                                                         "copy_rel_max": float(rel2.max()),
                                                         "routes_rel_diff": float(d)})
