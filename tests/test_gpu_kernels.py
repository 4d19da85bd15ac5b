"""Per-kernel parity of the HIP path against the oracle, through the C ABI.

Bar: routing ids, offsets, permutations, permuted rows and fp8 activation
codes/scales bit-exact; routing weights within 1e-5 relative; GEMM / combine
outputs within the row-normalised tolerance of their dtype (bf16 1e-2, fp8
2e-2, f32 1e-4), bit-exact on exact-arithmetic inputs; sentinel rows exactly 0.
"""
import numpy as np
import pytest
import torch

from helpers import TOL, np32, npu8, row_rel_err, say
from oracle import e4m3, gemm as ogemm, layer as olayer, routing as orouting
from workloads import quantize_weight_blocks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    import grouped_gemm_histogram_amd as g
    g.load()
    return g


# ------------------------------------------------------------------------------------ routing

ROUTE_CASES = [(1, 1, 1), (37, 8, 2), (500, 32, 4), (300, 64, 8), (257, 65, 3), (256, 128, 8),
               (129, 256, 8), (64, 1000, 16), (33, 1024, 16), (4096, 32, 4), (8192, 256, 8)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_route_topk(T, E, k, ties):
    say(f"route T={T} E={E} k={k} ties={ties}")
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        lg = (np.round(lg * 2) / 2).astype(np.float32)
        lg[lg == 0] = np.where(rng.random(np.count_nonzero(lg == 0)) < 0.5, -0.0, 0.0)
    g = ops()
    lt = torch.from_numpy(lg).to(DEV)
    for nv in (-1, (T * k) // 3, 0):
        for renorm in (True, False):
            ids, w = g.route_topk(lt, k, nv, renorm)
            rid, rw = orouting.route_topk(lg, k, nv, renorm)
            torch.cuda.synchronize()
            assert np.array_equal(ids.cpu().numpy(), rid), (nv, renorm)
            np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


# ------------------------------------------------------------------------------------ offsets

# R <= 1024 runs the single-workgroup kernel; larger R the three-kernel chunked path, in
# chunks of 256 rows up to 16384 rows and of 1024 rows beyond
OFFSET_CASES = [(1, 1), (100, 3), (1000, 8), (1024, 32), (1024, 1024), (64, 1024), (700, 256),
                (1025, 8), (1300, 5), (4096, 129), (16384, 128), (16384, 32), (16384, 1024), (16385, 8),
                (65536, 256), (65536, 1), (17000, 1024), (70000, 1024), (70000, 8), (40000, 1024),
                (5000, 1024), (3000, 1)]


@pytest.mark.parametrize("R,E", OFFSET_CASES)
def test_build_offsets(R, E):
    say(f"offsets R={R} E={E}")
    rng = np.random.default_rng(R + 3 * E)
    ids = rng.integers(0, E + 1, R).astype(np.int32)
    ids[rng.random(R) < 0.03] = -5
    ids[rng.random(R) < 0.03] = E + 11
    g = ops()
    off, sr, rp = g.build_offsets(torch.from_numpy(ids).to(DEV), E)
    roff, rsr, rrp = orouting.build_offsets(ids, E)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sr.cpu().numpy(), rsr)
    assert np.array_equal(rp.cpu().numpy(), rrp)


@pytest.mark.parametrize("pattern", ["one_expert", "all_sentinel", "one_hot", "last_expert"])
@pytest.mark.parametrize("R", [5000, 900])
def test_build_offsets_degenerate(pattern, R):
    say(f"offsets degenerate {pattern} R={R}")
    E = 64
    if pattern == "one_expert":
        ids = np.full(R, 17, np.int32)
    elif pattern == "all_sentinel":
        ids = np.full(R, E, np.int32)
    elif pattern == "one_hot":
        ids = np.arange(R, dtype=np.int32) % E
    else:
        ids = np.where(np.arange(R) % 3 == 0, E - 1, E).astype(np.int32)
    g = ops()
    off, sr, rp = g.build_offsets(torch.from_numpy(ids).to(DEV), E)
    roff, rsr, rrp = orouting.build_offsets(ids, E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sr.cpu().numpy(), rsr)
    assert np.array_equal(rp.cpu().numpy(), rrp)


def test_build_offsets_empty():
    g = ops()
    off, sr, rp = g.build_offsets(torch.empty(0, dtype=torch.int32, device=DEV), 8)
    assert off.cpu().tolist() == [0] * 9


# ------------------------------------------------------------------------------------ permute

def _routing(T, E, k, nv, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orouting.route_topk(lg, k, nv)
    off, sr, rp = orouting.build_offsets(ids.reshape(-1), E)
    return ids, w, off, sr, rp


@pytest.mark.parametrize("dtype,H", [(torch.bfloat16, 2880), (torch.bfloat16, 8), (torch.float32, 132),
                                     (torch.float32, 4), (torch.bfloat16, 7168)])
def test_permute_copy(dtype, H):
    say(f"permute copy {dtype} H={H}")
    T, E, k = 300, 16, 3
    ids, w, off, sr, rp = _routing(T, E, k, 700, 1)
    R = T * k
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(2)).to(dtype)
    g = ops()
    out = torch.full((R, H), float("nan"), dtype=dtype, device=DEV)
    g.permute(x.to(DEV), torch.from_numpy(sr).to(DEV), torch.from_numpy(off).to(DEV), k, out=out)
    got = out.cpu()
    ref = olayer.permute_rows(x.view(torch.int16).numpy() if dtype == torch.bfloat16
                              else x.view(torch.int32).numpy(), sr, off, k)
    V = int(off[-1])
    bits = got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(bits[:V], ref)
    assert torch.isnan(got[V:].float()).all()          # sentinel tail never written


def _sweep_rows():
    """bf16 rows whose 128-groups each hold 448*2^m plus sweep values * 2^m (scale = 2^m exactly)."""
    # every non-negative bf16 value up to 448, both signs, and their 2^m multiples
    bits = np.arange(0, 0x43E1, dtype=np.uint32)           # 0x43E0 is 448.0 in bf16
    vals = (bits << 16).view(np.float32)
    vals = vals[(vals <= 448.0) & ((vals == 0) | (vals >= 2.0 ** -100))]   # no fp32 denormals
    vals = np.concatenate([vals, -vals])
    groups = []
    for m in (-3, 0, 5):
        for i in range(0, len(vals), 127):
            grp = np.zeros(128, np.float32)
            chunk = vals[i:i + 127]
            grp[0] = 448.0
            grp[1:1 + len(chunk)] = chunk
            groups.append(grp * np.float32(2.0 ** m))
    flat = np.concatenate(groups)
    pad = (-len(flat)) % 512
    return np.concatenate([flat, np.zeros(pad, np.float32)]).reshape(-1, 512)


@pytest.mark.parametrize("case", ["random", "sweep"])
def test_permute_quant_fp8(case):
    say(f"permute quant fp8 {case}")
    if case == "sweep":
        xf = _sweep_rows()
        T, H = xf.shape
        x = torch.from_numpy(xf).to(torch.bfloat16)
        assert np.array_equal(x.float().numpy(), xf)          # all sweep values exact in bf16
        k, E = 1, 1
        ids = np.zeros((T, 1), np.int32)
        off, sr, rp = orouting.build_offsets(ids.reshape(-1), E)
    else:
        T, H, E, k = 200, 7168, 32, 8
        ids, w, off, sr, rp = _routing(T, E, k, 1500, 3)
        x = (torch.randn(T, H, generator=torch.Generator().manual_seed(4)) *
             torch.exp(torch.randn(T, 1, generator=torch.Generator().manual_seed(5)))).to(torch.bfloat16)
        x[3, :128] = 0                                        # all-zero group: scale 1
    R = T * k
    g = ops()
    q, s = g.permute(x.to(DEV), torch.from_numpy(sr).to(DEV), torch.from_numpy(off).to(DEV), k,
                     out_dtype=torch.float8_e4m3fn)
    torch.cuda.synchronize()
    xq, xs = olayer.quant128(x.float().numpy())
    V = int(off[-1])
    rq = olayer.permute_rows(xq, sr, off, k)
    rs = olayer.permute_rows(xs, sr, off, k)
    gq = npu8(q)[:V]
    gs = np.ascontiguousarray(s.cpu().numpy().T[:V])   # block-major [H/128, R] -> [R, H/128]
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, (bad[:5], gq[tuple(bad[0])], rq[tuple(bad[0])])
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
    if case == "sweep":
        # every code the encoder can produce appears
        assert len(np.unique(gq)) >= 250


# ------------------------------------------------------------------------------------ grouped GEMM

def _segments(M, E, V, seed, empty=(1,)):
    """offsets over M rows with V valid rows, ragged loads, some experts empty."""
    rng = np.random.default_rng(seed)
    wts = rng.random(E) + 0.2
    for e in empty:
        if e < E:
            wts[e] = 0
    cnt = np.floor(wts / wts.sum() * V).astype(np.int64)
    cnt[np.argmax(wts)] += V - cnt.sum()
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(cnt)
    assert off[-1] == V
    return off


GEMM_CASES = [
    # dtype, M, V, E, N, K, epilogue
    ("bf16", 1000, 900, 6, 400, 200, "silu_mul"),
    ("bf16", 1000, 1000, 6, 384, 256, "none"),
    ("bf16", 777, 500, 9, 2 * 456, 712, "silu_mul"),
    ("bf16", 640, 640, 3, 200, 136, "none"),
    ("bf16", 300, 0, 4, 128, 64, "silu_mul"),
    # output widths whose last 12-column run straddles the row end
    ("bf16", 900, 850, 5, 2 * 1408, 384, "silu_mul"),
    ("bf16", 700, 700, 3, 1412 - 4, 256, "none"),
    ("bf16", 500, 480, 4, 2 * 104, 192, "silu_mul"),
    # no epilogue, N = 2880 (15 weight tiles of 192); up to 1024 experts in one launch
    ("bf16", 1300, 1250, 4, 2880, 192, "none"),
    ("bf16", 9000, 8900, 1022, 200, 64, "none"),
    ("bf16", 9000, 8900, 1024, 200, 64, "none"),
    ("f32", 500, 420, 5, 2 * 100, 96, "silu_mul"),
    ("f32", 500, 500, 5, 132, 68, "none"),
    # decode-size launches (at most 8 rows per expert): 16-row tiles, ragged N and K tails
    ("bf16", 40, 40, 6, 400, 200, "silu_mul"),
    ("bf16", 60, 55, 8, 136, 72, "none"),
    ("bf16", 12, 10, 8, 136, 72, "none"),                     # narrow decode tiles (<= 2 rows/expert)
    ("bf16", 16, 9, 4, 2 * 1408, 384, "silu_mul"),
    # 8 to 32 rows per expert: the mid-size tiles (32 rows), ragged N and K tails
    ("bf16", 600, 560, 32, 400, 200, "silu_mul"),
    ("bf16", 700, 690, 24, 1400, 264, "none"),
    ("bf16", 2000, 1990, 64, 2 * 456, 712, "silu_mul"),
]


@pytest.mark.parametrize("dt,M,V,E,N,K,epi", GEMM_CASES)
def test_grouped_gemm(dt, M, V, E, N, K, epi):
    say(f"gemm {dt} M={M} V={V} E={E} N={N} K={K} {epi}")
    if dt == "bf16" and 8 * E < M <= 32 * E:
        assert ops().grouped_gemm_tile_shape(torch.bfloat16, epi, M, E)[0] == 32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(M + N + K)
    A = torch.randn(M, K, generator=gen).to(tdt)
    B = (torch.randn(E, N, K, generator=gen) * 0.05).to(tdt)
    off = _segments(M, E, V, M + E)
    g = ops()
    n_out = N // 2 if epi == "silu_mul" else N
    C = torch.full((M, n_out), float("nan"), dtype=tdt, device=DEV)
    g.grouped_gemm(A.to(DEV), B.to(DEV), torch.from_numpy(off).to(DEV), epi, out=C)
    got = np32(C)
    ref = ogemm.grouped_gemm(A.float().numpy(), B.float().numpy(), off, epi)
    assert np.all(got[V:] == 0)
    err = row_rel_err(got[:V], ref[:V])
    say(f"  err {err:.3e}")
    assert err <= TOL[dt]
    # determinism
    C2 = torch.empty_like(C)
    g.grouped_gemm(A.to(DEV), B.to(DEV), torch.from_numpy(off).to(DEV), epi, out=C2)
    idt = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(C.cpu().view(idt), C2.cpu().view(idt))


def test_grouped_gemm_exact_bf16():
    say("gemm exact bf16")
    M, E, N, K = 700, 5, 320, 512
    gen = torch.Generator().manual_seed(11)
    A = torch.randint(-4, 5, (M, K), generator=gen).to(torch.bfloat16)
    B = torch.randint(-4, 5, (E, N, K), generator=gen).to(torch.bfloat16)
    off = _segments(M, E, 650, 12)
    g = ops()
    C = g.grouped_gemm(A.to(DEV), B.to(DEV), torch.from_numpy(off).to(DEV), "none", out_dtype=torch.float32)
    ref = ogemm.grouped_gemm(A.float().numpy(), B.float().numpy(), off)
    assert np.array_equal(C.cpu().numpy(), ref.astype(np.float32))


def _fp8_operands(M, E, N, K, seed, exact=False):
    gen = torch.Generator().manual_seed(seed)
    if exact:
        a_codes = e4m3.encode(torch.randint(-4, 5, (M, K), generator=gen).float().numpy())
        a_s = (2.0 ** torch.randint(-2, 3, (M, K // 128), generator=gen).float()).numpy()
        b_codes = e4m3.encode(torch.randint(-4, 5, (E, N, K), generator=gen).float().numpy())
        b_s = (2.0 ** torch.randint(-3, 1, (E, N // 128, K // 128), generator=gen).float()).numpy()
        return a_codes, a_s.astype(np.float32), b_codes, b_s.astype(np.float32)
    a = torch.randn(M, K, generator=gen) * torch.exp(torch.randn(M, 1, generator=gen))
    a_codes, a_s = olayer.quant128(a.numpy())
    bq, bs = [], []
    for e in range(E):
        q, s = quantize_weight_blocks(torch.randn(N, K, generator=gen) * 0.02)
        bq.append(q.view(torch.uint8).numpy())
        bs.append(s.numpy())
    return a_codes, a_s, np.stack(bq), np.stack(bs)


def _u8_to_fp8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(DEV)


@pytest.mark.parametrize("M,V,E,N,K,epi,out", [
    (600, 520, 5, 512, 384, "silu_mul", "fp8"),
    (600, 600, 5, 512, 384, "silu_mul", "bf16"),
    (600, 480, 7, 384, 256, "none", "bf16"),
    (300, 0, 3, 256, 128, "silu_mul", "fp8"),
    (600, 570, 5, 512, 128, "silu_mul", "fp8"),
    (600, 590, 5, 384, 128, "none", "bf16"),
    # decode sizes (at most 8 rows per expert): 16-row tiles; fp8 output keeps 128-column tiles
    (40, 40, 6, 512, 384, "silu_mul", "bf16"),
    (40, 33, 6, 512, 384, "silu_mul", "f32"),
    (30, 25, 5, 384, 256, "none", "bf16"),
    (20, 18, 4, 512, 256, "silu_mul", "fp8"),
])
def test_grouped_gemm_fp8(M, V, E, N, K, epi, out):
    say(f"gemm fp8 M={M} V={V} E={E} N={N} K={K} {epi} -> {out}")
    aq, as_, bq, bs = _fp8_operands(M, E, N, K, M + N)
    off = _segments(M, E, V, E + 7)
    g = ops()
    odt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16, "f32": torch.float32}[out]
    n_out = N // 2 if epi == "silu_mul" else N
    C = torch.full((M, n_out), float("nan"), dtype=torch.float32, device=DEV).to(odt)
    res = g.grouped_gemm(_u8_to_fp8(aq), _u8_to_fp8(bq), torch.from_numpy(off).to(DEV), epi,
                         a_scales=torch.from_numpy(np.ascontiguousarray(as_.T)).to(DEV),
                         b_scales=torch.from_numpy(bs).to(DEV), out_dtype=odt, out=C)
    if out == "fp8":
        C, Cs = res
        gq, gs = npu8(C), Cs.cpu().numpy().T   # block-major -> [M, N_out/128]
        rd, rq, rs = ogemm.grouped_gemm(aq, bq, off, epi, as_, bs, out_fp8=True)
        assert np.all(gq[V:] == 0) and np.all(gs[V:] == 1.0)
        if V:
            # The code is decided in fp32 on both sides, but from h accumulated in
            # fp32 (GPU) vs float64 (oracle): a value within rounding noise of an
            # e4m3 midpoint may land one step apart.  Scales follow amax closely.
            np.testing.assert_allclose(gs[:V], rs[:V], rtol=2e-4)
            # In scale units (|code value| <= 448): the two codes may differ by one
            # e4m3 step at that magnitude plus the accumulation noise, which is
            # relative to the group max (448), not to the value itself.
            dg, dr = e4m3.decode(gq[:V]), e4m3.decode(rq[:V])
            mag = np.maximum(np.abs(dg), np.abs(dr))
            ulp = np.where(mag >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3),
                           2.0 ** -9)
            diff = np.abs(dg - dr)
            flips = np.count_nonzero(diff)
            say(f"  codes that differ: {flips} of {diff.size}; max diff/(ulp + noise) "
                f"{(diff / (ulp + 448 * 2e-4)).max():.3f}")
            assert np.all(diff <= ulp + 448 * 2e-4) and flips <= 0.01 * diff.size
    else:
        got = np32(C)
        ref = ogemm.grouped_gemm(aq, bq, off, epi, as_, bs)
        assert np.all(got[V:] == 0)
        err = row_rel_err(got[:V], ref[:V])
        say(f"  err {err:.3e}")
        assert err <= TOL["fp8"]


def test_grouped_gemm_fp8_exact():
    say("gemm fp8 exact")
    M, E, N, K = 400, 4, 256, 512
    aq, as_, bq, bs = _fp8_operands(M, E, N, K, 21, exact=True)
    off = _segments(M, E, 380, 22)
    g = ops()
    C = g.grouped_gemm(_u8_to_fp8(aq), _u8_to_fp8(bq), torch.from_numpy(off).to(DEV), "none",
                       a_scales=torch.from_numpy(np.ascontiguousarray(as_.T)).to(DEV),
                       b_scales=torch.from_numpy(bs).to(DEV), out_dtype=torch.float32)
    ref = ogemm.grouped_gemm(aq, bq, off, "none", as_, bs)
    assert np.array_equal(C.cpu().numpy(), ref.astype(np.float32))


# ------------------------------------------------------------------------------------ multi-tile GEMM

def _offsets_from_counts(cnt):
    off = np.zeros(len(cnt) + 1, np.int32)
    off[1:] = np.cumsum(cnt)
    return off


@pytest.mark.parametrize("epi", ["none", "silu_mul"])
def test_grouped_gemm_many_m_tiles(epi):
    """Experts of 961, 1300 and 2500 rows: 6, 7 and 14 m-tiles of 192 rows, so the tile order's
    blocks of m-tiles come in several full blocks plus a partial one; compared whole."""
    cnt = [961, 1300, 2500]
    off = _offsets_from_counts(cnt)
    M, E, N, K = int(off[-1]) + 37, 3, 2880, 640
    say(f"gemm many m-tiles {epi}: M_e={cnt} N={N} K={K}")
    gen = torch.Generator().manual_seed(41)
    A = torch.randint(-4, 5, (M, K), generator=gen).to(torch.bfloat16)
    B = torch.randint(-4, 5, (E, N, K), generator=gen).to(torch.bfloat16)
    g = ops()
    if epi == "none":
        # integer operands: every partial sum is exact in fp32, so the result is bit-exact
        C = g.grouped_gemm(A.to(DEV), B.to(DEV), torch.from_numpy(off).to(DEV), "none", out_dtype=torch.float32)
        ref = ogemm.grouped_gemm(A.float().numpy(), B.float().numpy(), off)
        assert np.array_equal(C.cpu().numpy(), ref.astype(np.float32))
    else:
        Bs = (B.float() * 2.0 ** -6).to(torch.bfloat16)        # keeps silu's argument moderate
        C = g.grouped_gemm(A.to(DEV), Bs.to(DEV), torch.from_numpy(off).to(DEV), "silu_mul")
        ref = ogemm.grouped_gemm(A.float().numpy(), Bs.float().numpy(), off, "silu_mul")
        got = np32(C)
        V = int(off[-1])
        assert np.all(got[V:] == 0)
        err = row_rel_err(got[:V], ref[:V])
        say(f"  err {err:.3e}")
        assert err <= TOL["bf16"]


def _exact_fp8(M, E, N, K, seed):
    gen = torch.Generator().manual_seed(seed)
    a_codes = e4m3.encode(torch.randint(-4, 5, (M, K), generator=gen).float().numpy())
    a_s = (2.0 ** torch.randint(-2, 3, (M, K // 128), generator=gen).float()).numpy().astype(np.float32)
    b_codes = e4m3.encode(torch.randint(-4, 5, (E, N, K), generator=gen).float().numpy())
    b_s = (2.0 ** torch.randint(-3, 1, (E, N // 128, K // 128), generator=gen).float()).numpy().astype(np.float32)
    return a_codes, a_s, b_codes, b_s


# Launches with more than two rounds of the persistent grid (256 workgroups on MI355X) and
# many K slices, so workgroups run several tiles each: the LDS stage rotation that carries
# over from one tile to the next is exercised everywhere.
# Integer operands (fp8: small-integer codes with power-of-two scales) make every partial sum
# exact in fp32, so the whole output is compared bit for bit, and a rerun must match it.
MULTI_TILE = [
    # dtype, gathered, T (token rows), k, E, N, K
    ("bf16", False, 16384, 1, 32, 1152, 1024),   # 32 x 3 m-tiles x 6 n-tiles = 576 tiles, 16 slices
    ("bf16", True, 4096, 4, 32, 1152, 1024),
    ("fp8", False, 16384, 1, 32, 1280, 2048),    # 128x256 tiles: ~32 x 4 x 5 tiles, 16 slices
    ("fp8", True, 4096, 4, 32, 1280, 2048),
    # one and three 128-deep fp8 slices per tile (the pipeline's first and last slice
    # coincide, or an odd count after the pairs), several tiles per workgroup
    ("fp8", False, 16384, 1, 32, 1280, 128),
    ("fp8", True, 4096, 4, 32, 1280, 384),
]


@pytest.mark.parametrize("dt,gathered,T,k,E,N,K", MULTI_TILE)
def test_grouped_gemm_multi_round_exact(dt, gathered, T, k, E, N, K):
    say(f"gemm multi-round exact {dt} gathered={gathered} T={T} k={k} E={E} N={N} K={K}")
    R = T * k
    ids, w, off, sr, rp = _routing(T, E, k, R - 300, 51 + k)
    V = int(off[-1])
    g = ops()
    d_off, d_sr = torch.from_numpy(off).to(DEV), torch.from_numpy(sr).to(DEV)
    if dt == "bf16":
        gen = torch.Generator().manual_seed(52)
        A = torch.randint(-4, 5, (T, K), generator=gen).to(torch.bfloat16)
        B = torch.randint(-4, 5, (E, N, K), generator=gen).to(torch.bfloat16)
        Ad, Bd = A.to(DEV), B.to(DEV)
        if gathered:
            run = lambda: g.grouped_gemm_gather(Ad, Bd, d_off, d_sr, k, "none", out_dtype=torch.float32)
            ref = ogemm.grouped_gemm(olayer.permute_rows(A.float().numpy(), sr, off, k), B.float().numpy(), off)
        else:
            run = lambda: g.grouped_gemm(Ad, Bd, d_off, "none", out_dtype=torch.float32)
            ref = ogemm.grouped_gemm(A.float().numpy(), B.float().numpy(), off)
    else:
        aq, as_, bq, bs = _exact_fp8(T, E, N, K, 53)
        Ad, Bd = _u8_to_fp8(aq), _u8_to_fp8(bq)
        d_as = torch.from_numpy(np.ascontiguousarray(as_.T)).to(DEV)
        d_bs = torch.from_numpy(bs).to(DEV)
        if gathered:
            run = lambda: g.grouped_gemm_gather(Ad, Bd, d_off, d_sr, k, "none", a_scales=d_as, b_scales=d_bs,
                                                out_dtype=torch.float32)
            ref = ogemm.grouped_gemm(olayer.permute_rows(aq, sr, off, k), bq, off, "none",
                                     olayer.permute_rows(as_, sr, off, k), bs)
        else:
            run = lambda: g.grouped_gemm(Ad, Bd, d_off, "none", a_scales=d_as, b_scales=d_bs,
                                         out_dtype=torch.float32)
            ref = ogemm.grouped_gemm(aq, bq, off, "none", as_, bs)
    C = run()
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    assert np.array_equal(got[:V], ref[:V].astype(np.float32))
    assert np.all(got[V:] == 0)
    C2 = run()
    assert torch.equal(C.cpu().view(torch.int32), C2.cpu().view(torch.int32))


# Launches of one, two and three 64-deep K slices with several tiles per workgroup: a
# tile's first slices land in stages that follow on from the previous tile's, here with
# fewer slices per tile than LDS stages; E = 63, empty experts (the last among them), experts of
# exactly 256 and 512 rows, ragged output widths.  Integer operands: bit-exact against the
# oracle.
SHORT_K_CASES = [
    # K, N, epilogue, gathered, E
    (64, 2304, "none", False, 32),
    (128, 2304, "silu_mul", False, 32),
    (192, 2304, "none", True, 32),
    (64, 1008, "silu_mul", True, 63),
    (320, 2880, "none", False, 63),
    (256, 2880, "silu_mul", True, 8),
]


@pytest.mark.parametrize("K,N,epi,gathered,E", SHORT_K_CASES)
def test_grouped_gemm_short_k_multi_tile(K, N, epi, gathered, E):
    g = ops()
    say(f"gemm short K={K} N={N} {epi} gathered={gathered} E={E}")
    gen = torch.Generator().manual_seed(K + N + E)
    T, k = (4096, 4) if gathered else (16384, 1)
    if gathered:
        ids, w, off, sr, rp = _routing(T, E, k, T * k - 123, K + E)
    else:
        # ragged loads summing to at most 16284 rows, with experts of 256 and 512 rows and
        # empty ones (including the last)
        wts = np.random.default_rng(E).random(E)
        wts[:3] = 0
        wts[E - 1] = 0
        cnt = np.floor(wts / wts.sum() * (16284 - 768)).astype(np.int64)
        cnt[0], cnt[1] = 256, 512
        off = _offsets_from_counts(cnt)
        assert off[-1] <= 16284
    V = int(off[-1])
    A = torch.randint(-3, 4, (T, K), generator=gen).to(torch.bfloat16)
    B = torch.randint(-3, 4, (E, N, K), generator=gen).to(torch.bfloat16)
    if epi == "silu_mul":
        B = (B.float() * 2.0 ** -5).to(torch.bfloat16)
    d_off = torch.from_numpy(off).to(DEV)
    odt = torch.float32 if epi == "none" else torch.bfloat16
    n_out = N // 2 if epi == "silu_mul" else N
    C = torch.full((T * k, n_out), float("nan"), dtype=odt, device=DEV)
    if gathered:
        g.grouped_gemm_gather(A.to(DEV), B.to(DEV), d_off, torch.from_numpy(sr).to(DEV), k, epi, out_dtype=odt, out=C)
        ref = ogemm.grouped_gemm(olayer.permute_rows(A.float().numpy(), sr, off, k), B.float().numpy(), off, epi)
    else:
        g.grouped_gemm(A.to(DEV), B.to(DEV), d_off, epi, out_dtype=odt, out=C)
        ref = ogemm.grouped_gemm(A.float().numpy(), B.float().numpy(), off, epi)
    got = np32(C)
    assert np.all(got[V:] == 0)
    if epi == "none":
        assert np.array_equal(got[:V], ref[:V].astype(np.float32))
    else:
        err = row_rel_err(got[:V], ref[:V])
        say(f"  err {err:.3e}")
        assert err <= TOL["bf16"]


# ------------------------------------------------------------------------------------ gathered GEMM

GATHER_CASES = [
    # dtype, T, E, k, valid rows (-1: all), N, K, epilogue
    ("bf16", 300, 8, 4, -1, 2 * 456, 712, "silu_mul"),
    ("bf16", 257, 16, 2, 300, 384, 256, "none"),
    ("bf16", 64, 4, 2, 0, 128, 64, "silu_mul"),
    ("bf16", 700, 3, 1, -1, 400, 200, "silu_mul"),
    ("f32", 200, 6, 3, 450, 2 * 100, 96, "silu_mul"),
    ("bf16", 5, 16, 4, -1, 2 * 456, 712, "silu_mul"),         # decode tiles
    ("bf16", 30, 8, 2, 50, 384, 264, "none"),                 # decode tiles, K tail
    ("fp8", 200, 8, 4, 700, 512, 384, "silu_mul"),
    ("fp8", 150, 5, 2, -1, 384, 256, "none"),
]


@pytest.mark.parametrize("dt,T,E,k,nv,N,K,epi", GATHER_CASES)
def test_grouped_gemm_gather(dt, T, E, k, nv, N, K, epi):
    """Token rows read through sorted_rows: oracle parity on the permuted rows, zeros past V,
    and the same bits as permute + grouped_gemm."""
    say(f"gather gemm {dt} T={T} E={E} k={k} nv={nv} N={N} K={K} {epi}")
    ids, w, off, sr, rp = _routing(T, E, k, nv, T + N)
    R, V = T * k, int(off[-1])
    g = ops()
    n_out = N // 2 if epi == "silu_mul" else N
    d_off, d_sr = torch.from_numpy(off).to(DEV), torch.from_numpy(sr).to(DEV)
    kw = {}
    if dt == "fp8":
        aq, as_, bq, bs = _fp8_operands(T, E, N, K, T + N)
        A, B = _u8_to_fp8(aq), _u8_to_fp8(bq)
        kw = dict(a_scales=torch.from_numpy(np.ascontiguousarray(as_.T)).to(DEV),
                  b_scales=torch.from_numpy(bs).to(DEV))
        odt = torch.bfloat16
        ref = ogemm.grouped_gemm(olayer.permute_rows(aq, sr, off, k), bq, off, epi,
                                 olayer.permute_rows(as_, sr, off, k), bs)
    else:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        gen = torch.Generator().manual_seed(T + K)
        A = torch.randn(T, K, generator=gen).to(tdt)
        B = (torch.randn(E, N, K, generator=gen) * 0.05).to(tdt)
        ref = ogemm.grouped_gemm(olayer.permute_rows(A.float().numpy(), sr, off, k), B.float().numpy(), off, epi)
        A, B, odt = A.to(DEV), B.to(DEV), tdt
    C = torch.full((R, n_out), float("nan"), dtype=torch.float32, device=DEV).to(odt)
    g.grouped_gemm_gather(A, B, d_off, d_sr, k, epi, out=C, **kw)
    got = np32(C)
    assert np.all(got[V:] == 0)
    if V:
        err = row_rel_err(got[:V], ref[:V])
        say(f"  err {err:.3e}")
        assert err <= TOL[dt]
    # the unfused sequence gives the same bits
    if dt == "fp8":
        xp = torch.zeros(R, K, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
        xs = torch.ones(K // 128, R, dtype=torch.float32, device=DEV)
        xp[:V] = A[d_sr[:V].long() // k]
        xs[:, :V] = kw["a_scales"][:, d_sr[:V].long() // k]
        C2 = g.grouped_gemm(xp, B, d_off, epi, a_scales=xs, b_scales=kw["b_scales"], out_dtype=odt)
    else:
        C2 = g.grouped_gemm(g.permute(A, d_sr, d_off, k, out=torch.zeros(R, K, dtype=A.dtype, device=DEV)),
                            B, d_off, epi)
    idt = torch.int16 if odt == torch.bfloat16 else torch.int32
    assert torch.equal(C.cpu().view(idt), C2.cpu().view(idt))


@pytest.mark.parametrize("T", [400, 16])
def test_grouped_gemm_gather_exact_bf16(T):
    say(f"gather gemm exact bf16 T={T}")
    E, k, N, K = 6, 3, 256, 384
    ids, w, off, sr, rp = _routing(T, E, k, T * k - 20, 31)
    gen = torch.Generator().manual_seed(32)
    A = torch.randint(-4, 5, (T, K), generator=gen).to(torch.bfloat16)
    B = torch.randint(-4, 5, (E, N, K), generator=gen).to(torch.bfloat16)
    g = ops()
    C = g.grouped_gemm_gather(A.to(DEV), B.to(DEV), torch.from_numpy(off).to(DEV), torch.from_numpy(sr).to(DEV),
                              k, "none", out_dtype=torch.float32)
    V = int(off[-1])
    ref = ogemm.grouped_gemm(olayer.permute_rows(A.float().numpy(), sr, off, k), B.float().numpy(), off)
    got = C.cpu().numpy()
    assert np.array_equal(got[:V], ref.astype(np.float32)) and np.all(got[V:] == 0)


@pytest.mark.parametrize("T,H", [(333, 1024), (1, 128), (64, 7168)])
def test_quantize_rows(T, H):
    say(f"quantize rows T={T} H={H}")
    gen = torch.Generator().manual_seed(T + H)
    x = (torch.randn(T, H, generator=gen) * torch.exp(torch.randn(T, 1, generator=gen))).to(torch.bfloat16)
    x[T // 2, :128] = 0                                       # all-zero group: scale 1
    q, s = ops().quantize_rows(x.to(DEV))
    xq, xs = olayer.quant128(x.float().numpy())
    assert np.array_equal(npu8(q), xq)
    assert np.array_equal(np.ascontiguousarray(s.cpu().numpy().T).view(np.uint32), xs.view(np.uint32))


# ------------------------------------------------------------------------------------ combine

@pytest.mark.parametrize("ydt,odt,H,k", [(torch.bfloat16, torch.bfloat16, 2880, 4), (torch.float32, torch.float32, 132, 4),
                                         (torch.bfloat16, torch.float32, 64, 4), (torch.float32, torch.bfloat16, 4, 4),
                                         (torch.bfloat16, torch.bfloat16, 1096, 16)])
def test_combine(ydt, odt, H, k):
    say(f"combine {ydt}->{odt} H={H} k={k}")
    T, E = 333, (12 if k <= 12 else 20)
    ids, w, off, sr, rp = _routing(T, E, k, 1000, 9)
    R = T * k
    V = int(off[-1])
    y = torch.randn(R, H, generator=torch.Generator().manual_seed(10)).to(ydt)
    y[V:] = float("nan")                                   # sentinel rows are never read
    g = ops()
    out = g.unpermute_combine(y.to(DEV), torch.from_numpy(rp).to(DEV), torch.from_numpy(w).to(DEV),
                              torch.from_numpy(off).to(DEV), k, out_dtype=odt)
    got = np32(out)
    ref = olayer.combine(y.float().numpy().astype(np.float64), rp, ids.reshape(-1), w.reshape(-1), T, k, E)
    dead = (np.arange(T) * k) >= V
    assert np.all(got[dead] == 0)
    tol = 1e-2 if odt == torch.bfloat16 else 1e-5
    assert row_rel_err(got[~dead], ref[~dead]) <= tol


def test_combine_y_beyond_mall():
    """y larger than 256 MiB takes the launch with four column steps of loads in flight."""
    T, k, E, H = 1024, 16, 20, 8704
    R = T * k
    assert R * H * 2 > 256 << 20
    say(f"combine bf16 T={T} k={k} H={H} (y {R * H * 2 / 2**20:.0f} MiB)")
    ids, w, off, sr, rp = _routing(T, E, k, R - 1000, 11)
    V = int(off[-1])
    y = torch.randn(R, H, generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    y[V:] = float("nan")
    out = ops().unpermute_combine(y.to(DEV), torch.from_numpy(rp).to(DEV), torch.from_numpy(w).to(DEV),
                                  torch.from_numpy(off).to(DEV), k, out_dtype=torch.bfloat16)
    got = np32(out)
    ref = olayer.combine(y.float().numpy(), rp, ids.reshape(-1), w.reshape(-1), T, k, E)
    dead = (np.arange(T) * k) >= V
    assert np.all(got[dead] == 0)
    assert row_rel_err(got[~dead], ref[~dead]) <= 1e-2
