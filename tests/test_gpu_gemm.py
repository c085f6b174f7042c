"""GPU tests of the GEMM building block (nsg_gemm_nt) against a plain fp32
reference of the same product, through the C ABI."""
import pytest
import torch

import newton_schulz_gram_amd as nsg

pytestmark = pytest.mark.gpu

TOL = {torch.float16: 2e-3, torch.bfloat16: 1.2e-2, torch.float32: 2e-6}


def ref_nt(A, B, alpha=1.0, beta=0.0, Cin=None):
    a = A.float().contiguous()
    bt = B.float().transpose(1, 2).contiguous()
    v = alpha * torch.bmm(a, bt)
    if Cin is not None:
        v = v + beta * Cin.float()
    return v


def rel(x, y):
    return float((x.float() - y.float()).norm() / y.float().norm().clamp_min(1e-30))


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("MNK", [(256, 256, 256), (512, 768, 256), (256, 512, 1024), (1024, 768, 512)])
def test_general_gemm(dtype, MNK, tile):
    M, N, K = MNK
    g = torch.Generator(device="cuda").manual_seed(1)
    A = torch.randn(3, M, K, device="cuda", generator=g).to(dtype)
    B = torch.randn(3, N, K, device="cuda", generator=g).to(dtype)
    Cin = torch.randn(3, M, N, device="cuda", generator=g).to(dtype)
    out, out_t, _ = nsg.gemm_nt(A, B, alpha=0.5, beta=-1.25, Cin=Cin, transposed_out=True, tile=tile)
    torch.cuda.synchronize()
    ref = ref_nt(A, B, 0.5, -1.25, Cin)
    assert rel(out, ref) <= TOL[dtype]
    assert torch.equal(out_t, out.transpose(1, 2).contiguous())


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,K", [(256, 512), (768, 256), (1024, 1024)])
def test_symmetric_gemm_gram(dtype, n, K, tile):
    """X X^T on the lower-triangle tiles only, mirrored: exactly symmetric."""
    g = torch.Generator(device="cuda").manual_seed(2)
    X = torch.randn(2, n, K, device="cuda", generator=g).to(dtype)
    out, _, _ = nsg.gemm_nt(X, X, alpha=2.0, symmetric=True, tile=tile)
    torch.cuda.synchronize()
    assert torch.equal(out, out.transpose(1, 2))
    assert rel(out, ref_nt(X, X, 2.0)) <= TOL[dtype]


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_symmetric_quadratic_with_dual_store(dtype, tile):
    """Z = b R + c R R^T (R symmetric) and the second store Z + a I."""
    g = torch.Generator(device="cuda").manual_seed(3)
    n = 512
    X = torch.randn(1, n, 1024, device="cuda", generator=g) / 32
    R = (X @ X.transpose(1, 2)).to(dtype)
    R = ((R.float() + R.float().transpose(1, 2)) / 2).to(dtype)  # exactly symmetric
    Z, _, Q = nsg.gemm_nt(R, R, alpha=2.0315, beta=-4.775, Cin=R, symmetric=True, diag=3.4445, tile=tile)
    torch.cuda.synchronize()
    ref = ref_nt(R, R, 2.0315, -4.775, R)
    assert torch.equal(Z, Z.transpose(1, 2)) and torch.equal(Q, Q.transpose(1, 2))
    assert rel(Z, ref) <= TOL[dtype]
    eye = torch.eye(n, device="cuda", dtype=torch.bool).unsqueeze(0)
    assert torch.equal(Q[~eye], Z[~eye])
    refq = ref + 3.4445 * torch.eye(n, device="cuda")
    assert rel(Q, refq) <= TOL[dtype]


def test_gemm_rejects_unpadded_sizes():
    A = torch.zeros(1, 200, 256, device="cuda", dtype=torch.float16)
    with pytest.raises(nsg.NSGError):
        nsg.gemm_nt(A, A)


@pytest.mark.parametrize("tile", [128, 256])
def test_symmetric_product_of_distinct_operands_is_mirrored(tile):
    """Z (RZ) with RZ not exactly symmetric: only the lower triangle is computed
    and mirrored, so the output is exactly symmetric and equals the lower
    triangle of the full product."""
    g = torch.Generator(device="cuda").manual_seed(4)
    n = 768
    Z = torch.randn(2, n, n, device="cuda", generator=g).half()
    W = torch.randn(2, n, n, device="cuda", generator=g).half()
    out, _, _ = nsg.gemm_nt(Z, W, symmetric=True, tile=tile)
    torch.cuda.synchronize()
    ref = ref_nt(Z, W)
    low = torch.tril(torch.ones(n, n, device="cuda", dtype=torch.bool))
    assert torch.equal(out, out.transpose(1, 2))
    assert rel(out[:, low], ref[:, low]) <= TOL[torch.float16]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("kind,batch,n", [("sym", 3, 4096), ("sym", 2, 4352), ("gen", 5, 2048)])
def test_tile_schedule_covers_every_tile(dtype, kind, batch, n):
    """More 256 x 256 tiles than CUs and not a multiple of them (408, 306, 320
    tiles), and a triangle whose last row of 8 x 8-tile super-blocks is partial
    (17 tile rows): the persistent workgroups must produce every tile once."""
    g = torch.Generator(device="cuda").manual_seed(7)
    K = 256
    A = torch.randn(batch, n, K, device="cuda", generator=g).to(dtype)
    if kind == "sym":
        out, _, _ = nsg.gemm_nt(A, A, symmetric=True, tile=256)
        torch.cuda.synchronize()
        assert torch.equal(out, out.transpose(1, 2))
        ref = ref_nt(A, A)
    else:
        B = torch.randn(batch, n, K, device="cuda", generator=g).to(dtype)
        out, _, _ = nsg.gemm_nt(A, B, tile=256)
        torch.cuda.synchronize()
        ref = ref_nt(A, B)
    assert rel(out, ref) <= TOL[dtype]
    # no tile left unwritten or mixed up: every 256 x 256 block matches on its own
    d = (out.float() - ref).view(batch, n // 256, 256, n // 256, 256).norm(dim=(2, 4))
    r = ref.view(batch, n // 256, 256, n // 256, 256).norm(dim=(2, 4))
    assert float((d / r).max()) <= 4 * TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_several_tiles_per_workgroup_with_cin_and_kmajor(dtype):
    """Launches with more tiles than CUs (each workgroup runs several tiles,
    loading the next tile's first stage during an epilogue): a symmetric
    product with Cin and the +diag second store (40 x 10 tiles), and a general
    product with a K-major B and Cin (12 x 24 tiles), every 256 x 256 block
    against the fp32 reference and the K-major one bit for bit against the
    row-major one."""
    g = torch.Generator(device="cuda").manual_seed(11)
    b, n, K = 40, 1024, 512
    A = torch.randn(b, n, K, device="cuda", generator=g).to(dtype)
    C = torch.randn(b, n, n, device="cuda", generator=g)
    C = (C + C.transpose(1, 2)).to(dtype)
    out, _, out_d = nsg.gemm_nt(A, A, alpha=0.5, beta=-0.25, Cin=C, symmetric=True, diag=1.5, tile=256)
    torch.cuda.synchronize()
    ref = ref_nt(A, A, 0.5, -0.25, C)
    d = (out.float() - ref).view(b, n // 256, 256, n // 256, 256).norm(dim=(2, 4))
    r = ref.view(b, n // 256, 256, n // 256, 256).norm(dim=(2, 4))
    assert float((d / r).max()) <= 4 * TOL[dtype]
    # the second store is v + 1.5 I rounded once: off the diagonal it equals
    # the first, on it the fp32 reference plus 1.5
    eye = torch.eye(n, device="cuda", dtype=torch.bool).unsqueeze(0).expand(b, n, n)
    assert torch.equal(out_d[~eye], out[~eye])
    dref = torch.diagonal(ref, dim1=1, dim2=2) + 1.5
    assert rel(torch.diagonal(out_d, dim1=1, dim2=2), dref) <= TOL[dtype]
    M, N = 768, 2048
    A2 = torch.randn(12, M, K, device="cuda", generator=g).to(dtype)
    B2 = torch.randn(12, N, K, device="cuda", generator=g).to(dtype)
    C2 = torch.randn(12, M, N, device="cuda", generator=g).to(dtype)
    o_row, _, _ = nsg.gemm_nt(A2, B2, alpha=2.0, beta=0.5, Cin=C2, tile=256)
    o_km, _, _ = nsg.gemm_nt(A2, B2.transpose(1, 2).contiguous(), alpha=2.0, beta=0.5, Cin=C2, tile=256,
                             b_kmajor=True)
    torch.cuda.synchronize()
    assert torch.equal(o_row, o_km)
    ref2 = ref_nt(A2, B2, 2.0, 0.5, C2)
    d2 = (o_row.float() - ref2).view(12, M // 256, 256, N // 256, 256).norm(dim=(2, 4))
    r2 = ref2.view(12, M // 256, 256, N // 256, 256).norm(dim=(2, 4))
    assert float((d2 / r2).max()) <= 4 * TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("n,K,batch", [(512, 768, 3), (1024, 2048, 2), (4352, 512, 1)])
def test_kmajor_symmetric_gram_matches_row_major(dtype, n, K, batch):
    """X X^T with X passed K-major (as X^T, K x n): the transposed LDS reads
    hand the MFMAs the same fragments as the row-major path, so the result is
    bit for bit the same (and exactly symmetric)."""
    g = torch.Generator(device="cuda").manual_seed(21)
    X = torch.randn(batch, n, K, device="cuda", generator=g).to(dtype)
    Xt = X.transpose(1, 2).contiguous()
    ref, _, _ = nsg.gemm_nt(X, X, alpha=0.75, symmetric=True, tile=256)
    out, _, _ = nsg.gemm_nt(Xt, Xt, alpha=0.75, symmetric=True, tile=256, a_kmajor=True, b_kmajor=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert rel(out, ref_nt(X, X, 0.75)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("MNK", [(512, 768, 256), (768, 2048, 512), (256, 4352, 1024)])
@pytest.mark.parametrize("both", [False, True])
def test_kmajor_general_matches_row_major(dtype, MNK, both):
    """A B^T with B (and A) passed K-major, with Cin and the transposed copy:
    bit for bit the row-major result."""
    M, N, K = MNK
    g = torch.Generator(device="cuda").manual_seed(22)
    A = torch.randn(2, M, K, device="cuda", generator=g).to(dtype)
    B = torch.randn(2, N, K, device="cuda", generator=g).to(dtype)
    Cin = torch.randn(2, M, N, device="cuda", generator=g).to(dtype)
    ref, ref_t, _ = nsg.gemm_nt(A, B, alpha=-0.5, beta=1.25, Cin=Cin, transposed_out=True, tile=256)
    Ak = A.transpose(1, 2).contiguous() if both else A
    out, out_t, _ = nsg.gemm_nt(Ak, B.transpose(1, 2).contiguous(), alpha=-0.5, beta=1.25, Cin=Cin,
                                transposed_out=True, tile=256, a_kmajor=both, b_kmajor=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(out_t, ref_t)
    assert rel(out, ref_nt(A, B, -0.5, 1.25, Cin)) <= TOL[dtype]


def test_kmajor_rejected_where_unsupported():
    A = torch.zeros(1, 512, 512, device="cuda", dtype=torch.float16)
    with pytest.raises(nsg.NSGError):   # A alone K-major
        nsg.gemm_nt(A, A, tile=256, a_kmajor=True)
    with pytest.raises(nsg.NSGError):   # symmetric with one K-major operand
        nsg.gemm_nt(A, A, symmetric=True, tile=256, b_kmajor=True)
    with pytest.raises(nsg.NSGError):   # 128 x 128 kernel
        nsg.gemm_nt(A, A, tile=128, b_kmajor=True)
    with pytest.raises(nsg.NSGError):   # fp32
        nsg.gemm_nt(A.float(), A.float(), tile=256, b_kmajor=True)


@pytest.mark.parametrize("dtype,big,ok", [(torch.float16, 65520.0, 65504.0),
                                          (torch.bfloat16, float.fromhex("0x1.ffp127"), float.fromhex("0x1.fep127"))])
@pytest.mark.parametrize("tile", [256])
def test_nonfinite_flag_at_the_rounding_threshold(dtype, big, ok, tile):
    """The status flag reports an output that is non-finite after rounding to
    the output dtype: the fp16 (bf16) overflow threshold 65520 (0x1.ffp127,
    halfway above the largest bf16, a tie that rounds to the even infinity)
    rounds to infinity, the largest finite values do not; NaN is reported."""
    n, K = 256, 256
    A = torch.zeros(4, n, K, device="cuda", dtype=torch.float32)
    A[:, 3, 5] = 1.0
    B = torch.zeros(4, n, K, device="cuda", dtype=torch.float32)
    B[:, 200, 5] = 1.0
    vals = [ok, big, -big, float("nan")]
    for g, v in enumerate(vals):
        A[g, 3, 5] = 1.0 if v == v else float("nan")
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    # alpha carries the value in fp32: V[3, 200] = alpha * 1 * 1
    outs = []
    for g, v in enumerate(vals):
        alpha = v if v == v else 1.0
        o, _, _ = nsg.gemm_nt(A[g:g + 1].to(dtype), B[g:g + 1].to(dtype), alpha=alpha, tile=tile, status=st[g:g + 1])
        outs.append(o)
    torch.cuda.synchronize()
    assert st.tolist() == [0, 1, 1, 1]
    assert torch.isfinite(outs[0].float()).all() and not torch.isfinite(outs[1].float()).all()
