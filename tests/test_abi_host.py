"""Host-side checks of libfp8gemm.so that need no GPU: every symbol the header
declares is exported, argument validation returns the documented codes without
launching, and the tile/split planner keeps its invariants."""
import ctypes
import os
import re

import pytest

import moe_grouped_gemm_fp32_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

CONFIG2 = [(m, n, k) for m in (64, 128, 4096)
           for (n, k) in ((2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048))]


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:const\s+char\s*\*|int64_t|size_t|int)\s+(fp8_\w+)\s*\(", text, re.M)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(fg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fg._SIGS), "binding and header disagree"


def test_status_strings_and_utilities():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert fg.status_string(code) and fg.status_string(code) != "unknown status"
    assert fg.status_string(-99) == "unknown status"
    assert fg.get_mk_alignment_for_contiguous_layout() == 128
    assert [fg.scale_ld(r) for r in (1, 4, 5, 2111, 2112)] == [4, 4, 8, 2112, 2112]


def test_tile_count_worked_example_from_pages():
    # deepep.org/zh/deepgemm, 核心优化技术 / 非对齐块大小: on 132 SMs, BLOCK_N=112 keeps
    # 128 busy where BLOCK_N=128 keeps 112 (M=256, N=7168, BLOCK_M=128)
    rows = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "unaligned_block_tiles.txt"))]
    rows = [r for r in rows if r]
    assert len(rows) == 2
    for M, N, bm, bn, busy in ([int(x) for x in r] for r in rows):
        assert min(fg.num_tiles(M, N, bm, bn), 132) == busy


P = ctypes.c_void_p


def _dense(A=1 << 20, lda=7168, sa=1 << 20, ld_sa=64, B=1 << 20, ldb=7168, sb=1 << 20, D=1 << 20, ldd=2112,
           M=64, N=2112, K=7168):
    mk = lambda v: P(v) if v else None
    return fg.lib().fp8_gemm_nt(mk(A), lda, mk(sa), ld_sa, mk(B), ldb, mk(sb), mk(D), ldd, M, N, K, None, 0, None)


def test_argument_validation_codes_without_launch():
    assert _dense(A=0) == -1 and _dense(sa=0) == -1 and _dense(D=0) == -1
    assert _dense(K=100) == -2 and _dense(N=0) == -2 and _dense(M=-1) == -2
    assert _dense(lda=7000) == -3 and _dense(ldb=7169) == -3 and _dense(ldd=2100) == -3
    assert _dense(ld_sa=63) == -3 and _dense(ld_sa=66) == -3
    assert _dense(A=(1 << 20) + 8) == -3 and _dense(D=(1 << 20) + 1) == -3
    assert _dense(M=0) == 0  # empty problem: nothing to do
    L = fg.lib()
    # contiguous: missing m_indices / bad G; masked: missing masked_m / G out of range
    args = (P(1 << 20), 7168, P(1 << 20), 64, P(1 << 20), 7168, P(1 << 20), P(1 << 20), 4096)
    assert L.fp8_grouped_gemm_nt_contiguous(*args, None, 64, 4096, 7168, 4, None, 0, None) == -1
    assert L.fp8_grouped_gemm_nt_contiguous(*args, P(1 << 20), 64, 4096, 7168, 0, None, 0, None) == -2
    assert L.fp8_grouped_gemm_nt_masked(*args, None, 4, 64, 4096, 7168, 32, None, 0, None) == -1
    assert L.fp8_grouped_gemm_nt_masked(*args, P(1 << 20), 1025, 64, 4096, 7168, 32, None, 0, None) == -2


def test_valid_call_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _dense() == -5
    mk = lambda v: P(v)
    na = fg.lib().fp8_gemm_nt_noalloc
    assert na(mk(1 << 20), 7168, mk(1 << 20), 64, mk(1 << 20), 7168, mk(1 << 20), mk(1 << 20), 2112, 64, 2112, 7168,
              None) == -5
    assert na(None, 7168, mk(1 << 20), 64, mk(1 << 20), 7168, mk(1 << 20), mk(1 << 20), 2112, 64, 2112, 7168,
              None) == -1
    assert fg.noalloc_scratch_bytes() == (32 << 20) + 16384


@pytest.fixture
def cus256():
    fg.set_num_cus(256)
    yield
    fg.set_num_cus(0)


@pytest.mark.parametrize("M,N,K", CONFIG2)
def test_planner_invariants_on_dense_shapes(cus256, M, N, K):
    cfg = fg.query_config(fg.KIND_DENSE, M, N, K)
    bm, bn, s = cfg["block_m"], cfg["block_n"], cfg["split_k"]
    tiles = fg.num_tiles(M, N, bm, bn)
    full = cfg["full_tiles"]
    assert 0 <= full <= tiles and (s > 1 or full == tiles)
    assert cfg["num_units"] == full + (tiles - full) * s
    if s > 1 and full > 0:  # whole tiles for the full rounds, one round of split units
        assert full % 256 == 0 and (tiles - full) * s <= 256
    nkb = K // 128
    assert 1 <= s <= nkb and (s == 1 or nkb % s == 0 or -(-nkb // s) * (s - 1) < nkb)
    # every split owns at least one K block
    kbps = -(-nkb // s)
    assert kbps * (s - 1) < nkb
    # the planner does not leave most CUs idle when K allows splitting
    if tiles < 64 and nkb >= 16:
        assert s > 1 and full == 0 and cfg["num_units"] >= 128
    assert cfg["grid"] <= cfg["num_units"] and cfg["grid"] <= 512
    # one round when the units fit on the CUs (no unit waits for a second round);
    # otherwise a multiple of 8, so the grid-stride loop keeps each workgroup's XCD
    if cfg["num_units"] <= 256:
        assert cfg["grid"] == cfg["num_units"]
    else:
        assert cfg["grid"] % 8 == 0
    ws = fg.workspace_size(fg.KIND_DENSE, M, N, K)
    assert (ws > 0) == (s > 1)
    if s > 1:
        assert ws >= (tiles - full) * s * bm * bn * 4 + (tiles - full) * 4
        # without a workspace the call falls back to no split
        assert fg.query_config(fg.KIND_DENSE, M, N, K, workspace_bytes=0)["split_k"] == 1


def test_planner_masked_and_contiguous(cus256):
    for G in (1, 2, 4, 8, 16):
        for N, K in ((4096, 7168), (7168, 2048)):
            cfg = fg.query_config(fg.KIND_MASKED, 4096, N, K, G, expected_m=256)
            assert cfg["block_m"] in (64, 128, 256)
            ws = fg.workspace_size(fg.KIND_MASKED, 4096, N, K, G, 256)
            assert (ws > 0) == (cfg["split_k"] > 1)
            # the workspace holds the live tiles of twice expected_m rows per group
            if cfg["split_k"] > 1:
                cap = G * -(-512 // cfg["block_m"]) * -(-N // cfg["block_n"])
                assert ws == 16384 + cap * cfg["split_k"] * cfg["block_m"] * cfg["block_n"] * 4
                assert cfg["full_tiles"] == 0
            # without a workspace the masked call does not split
            assert fg.query_config(fg.KIND_MASKED, 4096, N, K, G, 256, workspace_bytes=0)["split_k"] == 1
    cfg = fg.query_config(fg.KIND_CONTIGUOUS, 32768, 4096, 7168, 4)
    assert 128 % cfg["block_m"] == 0


def test_force_config_validation():
    L = fg.lib()
    bad = fg.Config(96, 64, 1, 0, 0)
    assert L.fp8_gemm_force_config(ctypes.byref(bad)) == -7
    bad = fg.Config(64, 64, 0, 0, 0)
    assert L.fp8_gemm_force_config(ctypes.byref(bad)) == -7
    auto = fg.query_config(fg.KIND_DENSE, 4096, 4096, 7168)
    with fg.force_config(64, 128, 2):
        assert fg.query_config(fg.KIND_DENSE, 100, 300, 1024)["block_n"] == 128
        assert fg.query_config(fg.KIND_DENSE, 4096, 4096, 7168)["block_m"] == 64
    # leaving the context restores automatic selection
    assert fg.query_config(fg.KIND_DENSE, 4096, 4096, 7168) == auto


def _quant(X=1 << 20, ldx=7168, dt=0, Q=1 << 20, ldq=7168, sa=1 << 20, ld_sa=64, M=64, K=7168):
    mk = lambda v: P(v) if v else None
    return fg.lib().fp8_quantize_1x128(mk(X), ldx, dt, mk(Q), ldq, mk(sa), ld_sa, M, K, None)


def test_quantize_argument_validation_without_launch():
    assert _quant(X=0) == -1 and _quant(Q=0) == -1 and _quant(sa=0) == -1
    assert _quant(K=100) == -2 and _quant(K=0) == -2 and _quant(M=-1) == -2
    assert _quant(dt=2) == -3 and _quant(ldx=7000) == -3 and _quant(ldx=7172) == -3
    assert _quant(dt=1, ldx=7172) != -3  # FP32 rows need only 16-byte alignment (4 elements)
    assert _quant(ldq=7100) == -3 and _quant(ld_sa=63) == -3 and _quant(ld_sa=66) == -3
    assert _quant(X=(1 << 20) + 8) == -3 and _quant(Q=(1 << 20) + 4) == -3 and _quant(sa=(1 << 20) + 2) == -3


def test_ue8m0_argument_validation_without_launch():
    L = fg.lib()
    P = ctypes.c_void_p
    good = dict(A=P(1 << 20), lda=512, sa=P(1 << 20), ld_sa=64, B=P(1 << 20), ldb=512, sb=P(1 << 20),
                D=P(1 << 20), ldd=256, M=64, N=256, K=512)

    def call(**kw):
        a = dict(good, **kw)
        return L.fp8_gemm_nt_ue8m0(a["A"], a["lda"], a["sa"], a["ld_sa"], a["B"], a["ldb"], a["sb"], a["D"],
                                   a["ldd"], a["M"], a["N"], a["K"], None, 0, None)
    assert call(A=None) == -1 and call(sb=None) == -1
    assert call(K=100) == -2 and call(N=0) == -2
    assert call(lda=500) == -3 and call(ld_sa=62) == -3 and call(ldd=100) == -3
    assert call(M=0) == 0  # nothing to do, nothing launched


def test_c_argument_validation_without_launch():
    L = fg.lib()
    P = ctypes.c_void_p

    def call(C=P(1 << 20), ldc=256):
        return L.fp8_gemm_nt_c(P(1 << 20), 512, P(1 << 20), 64, P(1 << 20), 512, P(1 << 20), C, ldc, P(1 << 20),
                               256, 64, 256, 512, None, 0, None)
    assert call(ldc=255) == -3                   # ldc < N
    assert call(C=P((1 << 20) + 1)) == -3        # not 2-byte aligned
    st = L.fp8_gemm_nt_c(P(1 << 20), 512, P(1 << 20), 64, P(1 << 20), 512, P(1 << 20), P(1 << 20), 256,
                         P(1 << 20), 256, 0, 256, 512, None, 0, None)
    assert st == 0                               # M == 0: nothing to do


def test_k_grouped_argument_validation_without_launch():
    L = fg.lib()
    base = dict(A=1 << 20, lda=4096, sa=1 << 20, ld_sa=4096, B=1 << 20, ldb=7168, sb=1 << 20, ld_sb=7168,
                D=1 << 20, ldd=7168, d_gstride=4096 * 7168, ks=[256, 128], M=4096, N=7168, acc=0)

    def call(**kw):
        a = dict(base, **kw)
        ks = a["ks"] or []
        arr = (ctypes.c_int32 * max(len(ks), 1))(*ks)
        G = kw.get("G", len(ks))
        return L.fp8_k_grouped_gemm_tn_contiguous(
            P(a["A"]), a["lda"], P(a["sa"]), a["ld_sa"], P(a["B"]), a["ldb"], P(a["sb"]), a["ld_sb"],
            P(a["D"]), a["ldd"], a["d_gstride"], ctypes.cast(arr, ctypes.c_void_p) if a["ks"] is not None else None,
            G, a["M"], a["N"], a["acc"], None)

    assert call(A=0) == -1 and call(sb=0) == -1 and call(D=0) == -1 and call(ks=None, G=2) == -1
    assert call(ks=[200]) == -2 and call(ks=[-128]) == -2 and call(M=0) == -2 and call(N=0) == -2
    assert call(G=0) == -2 and call(ks=[128] * 257) == -2
    assert call(lda=4095) == -3 and call(lda=4104) == -3 and call(ldb=7100) == -3
    assert call(ld_sa=4000) == -3 and call(ld_sb=7000) == -3 and call(ldd=7000) == -3
    assert call(d_gstride=4095 * 7168) == -3 and call(A=(1 << 20) + 8) == -3 and call(D=(1 << 20) + 2) == -3
    import torch
    if not torch.cuda.is_available():
        assert call() == -5 and call(ks=[0, 0]) == -5   # valid: stops at the device check


@pytest.mark.parametrize("name,a_kc,b_kc", [("fp8_gemm_tn", False, False), ("fp8_gemm_nn", True, False),
                                            ("fp8_gemm_tt", False, True), ("fp8_gemm_tn_ue8m0", False, False),
                                            ("fp8_gemm_nn_ue8m0", True, False), ("fp8_gemm_tt_ue8m0", False, True)])
def test_layout_argument_validation_without_launch(name, a_kc, b_kc):
    """Every argument error is reported before any device call; the leading-dimension rule
    follows each operand's layout (K-contiguous: ld >= K, K-major: ld >= rows)."""
    M, N, K = 4096, 7168, 2048
    fn = getattr(fg.lib(), name)
    base = dict(A=1 << 20, lda=K if a_kc else M, sa=1 << 20, ld_sa=M, B=1 << 20, ldb=K if b_kc else N,
                sb=1 << 20, D=1 << 20, ldd=N, M=M, N=N, K=K, ws=0, wsb=0)

    def call(**kw):
        a = dict(base, **kw)
        return fn(P(a["A"]), a["lda"], P(a["sa"]), a["ld_sa"], P(a["B"]), a["ldb"], P(a["sb"]), P(a["D"]), a["ldd"],
                  a["M"], a["N"], a["K"], P(a["ws"]) if a["ws"] else None, a["wsb"], None)

    assert call(A=0) == -1 and call(sb=0) == -1 and call(D=0) == -1
    assert call(K=100) == -2 and call(N=0) == -2 and call(M=-1) == -2
    assert call(lda=(K if a_kc else M) - 16) == -3 and call(ldb=(K if b_kc else N) + 8) == -3
    assert call(ld_sa=M - 4) == -3 and call(ldd=N - 1) == -3 and call(A=(1 << 20) + 8) == -3
    assert call(ws=(1 << 20) + 8, wsb=1 << 20) == -3   # the workspace is 16-byte aligned
    import torch
    if not torch.cuda.is_available():
        assert call() == -5   # valid: stops at the device check


def test_layout_planner_splits_few_row_shapes():
    """The TN / NN / TT plan: 256x256 tiles when they give at least half the CUs a tile and
    pad the output by at most a quarter; otherwise the 128x128, 64x128 or 128x64 tile and
    the K split of least modelled time. K is split (at least five K blocks a unit, no
    empty split) only as far as all units run in one round and the workspace holds the
    partials; no split without a workspace."""
    fg.set_num_cus(256)
    try:
        L = fg.KIND_LAYOUT
        big = fg.query_config(L, 4096, 7168, 16384)
        assert (big["block_m"], big["block_n"], big["split_k"]) == (256, 256, 1)
        assert fg.workspace_size(L, 4096, 7168, 16384) == 0
        mid = fg.query_config(L, 4096, 2112, 7168)     # 144 tiles of 256x256, N padded by 9%
        assert (mid["block_m"], mid["block_n"], mid["split_k"]) == (256, 256, 1)
        small = fg.query_config(L, 2048, 2048, 7168)   # 64 tiles of 256x256: 256 of 128x128
        assert (small["block_m"], small["block_n"], small["split_k"]) == (128, 128, 1)
        wide = fg.query_config(L, 128, 32768, 512)     # 128 tiles of 256x256 would double the rows
        assert (wide["block_m"], wide["split_k"]) == (128, 1)
        for M, N, K in [(64, 2112, 7168), (128, 7168, 2048), (128, 4096, 7168), (64, 7168, 16384)]:
            cfg = fg.query_config(L, M, N, K)
            bm, bn = cfg["block_m"], cfg["block_n"]
            assert (bm, bn) in ((128, 128), (64, 128), (128, 64)) and cfg["split_k"] > 1
            tiles = fg.num_tiles(M, N, bm, bn)
            assert cfg["num_units"] == tiles * cfg["split_k"] <= 256
            kbps = -(-(K // 128) // cfg["split_k"])
            assert kbps >= 5 and -(-(K // 128) // kbps) == cfg["split_k"]   # no empty split
            ws = fg.workspace_size(L, M, N, K)
            assert ws == 16384 + tiles * cfg["split_k"] * bm * bn * 4
            assert fg.query_config(L, M, N, K, workspace_bytes=ws) == cfg
            assert fg.query_config(L, M, N, K, workspace_bytes=0)["split_k"] == 1
        # a workspace too small for the chosen split: another plan whose partials fit it
        M, N, K = 64, 2112, 7168
        cfg = fg.query_config(L, M, N, K)
        half = fg.workspace_size(L, M, N, K) // 2
        small = fg.query_config(L, M, N, K, workspace_bytes=half)
        assert small != cfg and small["split_k"] > 1
        with fg.force_config(small["block_m"], small["block_n"], small["split_k"]):
            assert fg.workspace_size(L, M, N, K) <= half
        with fg.force_config(256, 256, 3):
            f = fg.query_config(L, 64, 2112, 7168)
            assert (f["block_m"], f["split_k"]) == (256, 3)
    finally:
        fg.set_num_cus(0)
    with pytest.raises(fg.Fp8GemmError):
        with fg.force_config(256, 64):
            pass


def test_swiglu_quantize_argument_validation_without_launch():
    fn = fg.lib().fp8_swiglu_quantize_1x128
    base = dict(H=1 << 20, ldh=4096, dt=0, mi=None, Q=1 << 20, ldq=2048, sa=1 << 20, ld_sa=64, M=64, F=2048)

    def call(**kw):
        a = dict(base, **kw)
        return fn(P(a["H"]), a["ldh"], a["dt"], P(a["mi"]) if a["mi"] else None, P(a["Q"]), a["ldq"], P(a["sa"]),
                  a["ld_sa"], a["M"], a["F"], None)

    assert call(H=0) == -1 and call(Q=0) == -1 and call(sa=0) == -1
    assert call(F=100) == -2 and call(F=0) == -2 and call(M=-1) == -2
    assert call(ldh=4000) == -3 and call(ldh=4100) == -3 and call(dt=7) == -3 and call(ldq=2047) == -3
    assert call(ld_sa=60) == -3 and call(mi=(1 << 20) + 2) == -3 and call(H=(1 << 20) + 8) == -3
    import torch
    if not torch.cuda.is_available():
        assert call() == -5 and call(M=0) == -5


PAGE_CITATION = re.compile(r"es\.news\.hada\.io|bquan\.live|deepep\.org|kirim\.ai|GeekNews topic")


def declaration_comments():
    """(function name, text of the comment block that documents it) for every function the
    header declares; declarations that follow one another share the comment above them."""
    text = open(HEADER).read()
    out, last_comment = [], ""
    pos = 0
    for m in re.finditer(r"/\*.*?\*/|^\s*(?:const\s+char\s*\*|int64_t|size_t|int)\s+(fp8_\w+)\s*\(", text, re.M | re.S):
        if m.group(0).lstrip().startswith("/*"):
            last_comment = m.group(0)
        else:
            out.append((m.group(1), last_comment))
        pos = m.end()
    return out


def test_every_declaration_cites_its_passage():
    """Each entry point's comment names the page passage that defines its operation, or says
    that it is a utility of this library with no counterpart on the pages, or (the
    no-allocation variant) names the callers it is for: those that cannot allocate."""
    decls = declaration_comments()
    assert {n for n, _ in decls} == set(declared_functions())
    flat = [(n, " ".join(c.replace("*", " ").split())) for n, c in decls]
    missing = [n for n, c in flat if not (PAGE_CITATION.search(c) or "no counterpart on the pages" in c
                                           or "cannot allocate" in c)]
    assert not missing, "declarations without a citation: %s" % missing


def test_packed_and_transform_argument_validation_without_launch():
    L = fg.lib()

    def dense(**kw):
        a = dict(A=1 << 20, lda=512, sa=1 << 20, ld_sa=64, B=1 << 20, ldb=512, sb=1 << 20, D=1 << 20, ldd=256,
                 M=64, N=256, K=512)
        a.update(kw)
        mk = lambda v: P(v) if v else None
        return L.fp8_gemm_nt_ue8m0_packed(mk(a["A"]), a["lda"], mk(a["sa"]), a["ld_sa"], mk(a["B"]), a["ldb"],
                                          mk(a["sb"]), mk(a["D"]), a["ldd"], a["M"], a["N"], a["K"], None, 0, None)
    assert dense(sa=0) == -1 and dense(K=100) == -2 and dense(ld_sa=62) == -3 and dense(M=0) == 0

    def tr(**kw):
        a = dict(sf=1 << 20, ld_sf=9, rows=300, nkb=9, act=1, pack=1, out=1 << 20, ld_out=300)
        a.update(kw)
        mk = lambda v: P(v) if v else None
        return L.fp8_transform_sf_into_required_layout(mk(a["sf"]), a["ld_sf"], a["rows"], a["nkb"], a["act"],
                                                       a["pack"], mk(a["out"]), a["ld_out"], None)
    assert tr(sf=0) == -1 and tr(out=0) == -1
    assert tr(nkb=0) == -2 and tr(rows=-1) == -2
    assert tr(ld_sf=8) == -3 and tr(ld_out=299) == -3 and tr(ld_out=302) == -3   # < rows; not a multiple of 4
    assert tr(act=0, ld_out=2) == -3 and tr(act=0, pack=0, ld_out=8) == -3      # < ceil(nkb/4); < nkb
    assert tr(sf=(1 << 20) + 2) == -3
    import torch
    if not torch.cuda.is_available():
        assert tr() == -5 and tr(act=0, ld_out=3) == -5


def test_plan_cache_follows_forced_configs_and_arguments():
    """The planner's per-thread cache returns the plan of the current arguments: forcing a
    configuration, releasing it, another CU count or workspace size each give the plan the
    planner computes for them."""
    fg.set_num_cus(256)
    try:
        M, N, K = 64, 2112, 7168
        auto = fg.query_config(fg.KIND_DENSE, M, N, K)
        assert fg.query_config(fg.KIND_DENSE, M, N, K) == auto
        with fg.force_config(128, 128, 3):
            f = fg.query_config(fg.KIND_DENSE, M, N, K)
            assert (f["block_m"], f["block_n"], f["split_k"]) == (128, 128, 3)
        with fg.force_config(64, 128, 2):
            f = fg.query_config(fg.KIND_DENSE, M, N, K)
            assert (f["block_m"], f["block_n"], f["split_k"]) == (64, 128, 2)
        assert fg.query_config(fg.KIND_DENSE, M, N, K) == auto
        assert fg.query_config(fg.KIND_DENSE, M, N, K, workspace_bytes=0)["split_k"] == 1
        fg.set_num_cus(64)
        assert fg.query_config(fg.KIND_DENSE, M, N, K)["grid"] <= 64
        fg.set_num_cus(256)
        assert fg.query_config(fg.KIND_DENSE, M, N, K) == auto
        # many shapes in turn (more than the cache holds) keep their own plans
        shapes = [(m, n, k) for m in (64, 128, 4096) for n, k in ((2112, 7168), (24576, 1536), (7168, 2048))]
        first = [fg.query_config(fg.KIND_DENSE, *sh) for sh in shapes]
        for _ in range(3):
            assert [fg.query_config(fg.KIND_DENSE, *sh) for sh in shapes] == first
    finally:
        fg.set_num_cus(0)

