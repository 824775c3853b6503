"""GPU parity of the M-grouped contiguous and masked FP8 GEMMs against the CPU oracle:
padding / dead rows keep the sentinel, live rows match the oracle, grouped results
equal the dense GEMM of each group, and the full-size MoE shapes on sampled rows."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import SENT, assert_bit_exact, bits_of, compare, forced_workspace_bytes, host, sample_rows

pytestmark = pytest.mark.gpu


def run_contig(c, forced=None):
    D = c["D"].clone()
    M, N, K, G = c["M"], c["N"], c["K"], c["G"]
    nbytes = fg.workspace_size(fg.KIND_CONTIGUOUS, M, N, K, G)
    if forced is not None and forced[2] > 1:
        nbytes = forced_workspace_bytes(fg.KIND_CONTIGUOUS, M, N, K, G, forced)
    work = torch.zeros(nbytes, dtype=torch.uint8, device=D.device) if nbytes else None
    if forced is None:
        fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"], work)
    else:
        with fg.force_config(*forced):
            fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"], work)
    torch.cuda.synchronize()
    return D


def run_masked(c, forced=None):
    D = c["D"].clone()
    args = (c["A"], c["sa"], c["B"], c["sb"], D, c["masked_m"], c["expected_m"])
    if forced is None:
        fg.fp8_grouped_gemm_nt_masked(*args)
    else:
        with fg.force_config(*forced):
            fg.fp8_grouped_gemm_nt_masked(*args)
    torch.cuda.synchronize()
    return D


def d_bits(c):
    return bits_of(c["D"])


@pytest.mark.parametrize("kind", ["normal", "e1", "e3"])
@pytest.mark.parametrize("tile", [None, (64, 64, 1), (128, 128, 1), (64, 128, 1), (128, 64, 1), (64, 64, 2),
                                  (128, 256, 1), (128, 256, 2), (64, 96, 1), (128, 96, 2)],
                         ids=lambda t: "auto" if t is None else "%dx%d_s%d" % t)
def test_contiguous_small_all_tiles(cuda_device, kind, tile):
    c = synth.contiguous_case([5, 128, 0, 130, 1, 300], 200, 384, seed=41, device=cuda_device, kind=kind)
    D = run_contig(c, tile)
    ref, S = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), d_bits(c))
    got = bits_of(D)
    pad = c["m_indices"].cpu().numpy() < 0
    assert np.all(got[pad] == SENT), "padding rows must keep their contents"
    compare(kind, got[~pad], ref[~pad], f"contiguous {kind} {tile}")


def test_contiguous_all_padding_block_and_dense_equivalence(cuda_device):
    c = synth.contiguous_case([100, 128, 256], 256, 512, seed=42, device=cuda_device)
    mi = c["m_indices"].clone()
    mi[128:256] = -1  # a whole 128-row block of padding
    c["m_indices"] = mi
    D = run_contig(c, (128, 128, 1))
    got = bits_of(D)
    mih = mi.cpu().numpy()
    assert np.all(got[mih < 0] == SENT)
    ref, _ = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), d_bits(c))
    compare("normal", got[mih >= 0], ref[mih >= 0], "contiguous with empty block")
    # a segment equals the dense GEMM of its rows with its expert's weights, bitwise
    seg = slice(256, 512)
    sa_seg = c["sa"][:, seg].contiguous()
    Dd = synth.sentinel_output((256, 256), cuda_device)
    with fg.force_config(128, 128, 1):
        fg.fp8_gemm_nt(c["A"][seg].contiguous(), sa_seg, c["B"][2].contiguous(), c["sb"][2].contiguous(), Dd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(Dd), got[seg])


@pytest.mark.parametrize("kind", ["normal", "e1", "e2"])
@pytest.mark.parametrize("tile", [None, (64, 64, 1), (64, 128, 1), (128, 128, 1), (256, 128, 1), (128, 256, 1)],
                         ids=lambda t: "auto" if t is None else "%dx%d_s%d" % t)
def test_masked_small_all_tiles(cuda_device, kind, tile):
    c = synth.masked_case(5, 256, 160, 384, seed=51, device=cuda_device, masked_m=[256, 0, 1, 179, 64],
                          kind=kind, expected_m=128)
    D = run_masked(c, tile)
    got = bits_of(D)
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), c["masked_m_list"], d_bits(c))
    for g, live in enumerate(c["masked_m_list"]):
        assert np.all(got[g, live:] == SENT), f"dead rows of group {g} were written"
        compare(kind, got[g, :live], ref[g, :live], f"masked {kind} {tile} group {g}")


def test_masked_full_group_equals_dense_and_empty_groups(cuda_device):
    c = synth.masked_case(3, 192, 256, 256, seed=52, device=cuda_device, masked_m=[192, 0, 0])
    D = run_masked(c, (64, 64, 1))
    got = bits_of(D)
    assert np.all(got[1:] == SENT)
    Dd = synth.sentinel_output((192, 256), cuda_device)
    with fg.force_config(64, 64, 1):
        fg.fp8_gemm_nt(c["A"][0], c["sa"][0], c["B"][0], c["sb"][0], Dd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(Dd), got[0])
    # every group empty: nothing is written at all
    c0 = synth.masked_case(2, 64, 128, 128, seed=53, device=cuda_device, masked_m=[0, 0])
    assert np.all(bits_of(run_masked(c0)) == SENT)


@pytest.mark.parametrize("G,rows,N,K", [(4, 8192, 4096, 7168), (8, 4096, 7168, 2048)])
def test_config3_contiguous_full_size_sampled(cuda_device, G, rows, N, K):
    c = synth.contiguous_case([rows] * G, N, K, seed=3000 + G, device=cuda_device)
    D = run_contig(c)
    got = bits_of(D)
    assert not np.any(got == SENT)
    rs = np.unique(np.concatenate([sample_rows(G * rows, 6, g) + 0 for g in range(1)] +
                                  [g * rows + sample_rows(rows, 3, g) for g in range(G)]))
    ref, _ = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), d_bits(c), rs, np.arange(N))
    compare("normal", got[rs], ref, f"config3 G={G}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_config4_masked_full_size_sampled(cuda_device, G, N, K):
    c = synth.masked_case(G, 4096, N, K, seed=4000 + G + N, device=cuda_device, expected_m=256)
    D = run_masked(c)
    mm = c["masked_m_list"]
    assert all(179 <= v <= 333 for v in mm)
    dead = torch.zeros(G, 4096, dtype=torch.bool, device=cuda_device)
    for g, live in enumerate(mm):
        dead[g, live:] = True
    Dv = D.view(torch.int16)
    assert bool((Dv[dead] == -1).all()), "dead rows must keep the sentinel"
    assert not bool((Dv[~dead] == -1).any()), "every live row must be written"
    rows = np.unique(np.concatenate([[0, 1, 178], np.random.default_rng(G).choice(179, 6, replace=False)]))
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm, d_bits(c), rows, np.arange(N))
    compare("normal", bits_of(D)[:, rows], ref, f"config4 G={G} N={N}")
    # per group: rows in [179, masked_m[g]) (the live rows beyond the common prefix,
    # in the later live tiles), including the last live row
    rng = np.random.default_rng(100 + G)
    for g in range(G):
        tail = np.arange(179, mm[g])
        pick = np.unique(np.concatenate([rng.choice(tail, min(4, len(tail)), replace=False), [mm[g] - 1]]))
        r1, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm, d_bits(c), pick, np.arange(N))
        compare("normal", bits_of(D)[g, pick], r1[g], f"config4 rows {list(pick)} of group {g}")


def test_config5_moe_ffn_pair(cuda_device):
    c1 = synth.moe_case(seed=5000, device=cuda_device, N=4096, K=7168)
    mi = c1["m_indices"]
    Mt = c1["M"]
    assert int((mi >= 0).sum()) == 4096 * 8 and Mt % 128 == 0
    D1 = run_contig(c1)
    pad = (mi < 0)
    D1v = D1.view(torch.int16)
    assert bool((D1v[pad] == -1).all()) and not bool((D1v[~pad] == -1).any())
    mih = mi.cpu().numpy()
    # sample rows from the most and least loaded experts and a few in between
    counts = np.array(c1["counts"])
    experts = list(np.argsort(counts)[[0, 1, 128, 254, 255]])
    rows = np.concatenate([np.nonzero(mih == e)[0][:3] for e in experts if counts[e] > 0] +
                          [np.nonzero(mih == e)[0][-2:] for e in experts if counts[e] > 0])
    rows = np.unique(rows)
    A1, sa1, mi1 = host(c1, "A", "sa", "m_indices")
    B1 = np.zeros((256, 1, 1), dtype=np.uint8)  # placeholder; only sampled experts are copied
    ref_rows = []
    for r in rows:
        e = int(mih[r])
        Bh = c1["B"][e].cpu().numpy()
        sbh = c1["sb"][e].cpu().numpy()
        b, _ = oracle.gemm_nt_sampled(A1, sa1, Bh, sbh, [r], np.arange(4096))
        ref_rows.append(b[0])
    compare("normal", bits_of(D1)[rows], np.stack(ref_rows), "moe gate+up")
    del B1
    # down projection on the SwiGLU of the gate+up output (harness glue, untimed)
    A2, sa2 = synth.swiglu_requant(D1.view(torch.bfloat16).float().nan_to_num(0.0), mi)
    g2 = synth.make_generator(5001, cuda_device)
    B2 = torch.empty(256, 7168, 2048, dtype=torch.uint8, device=cuda_device)
    sb2 = torch.empty(256, 56, 16, dtype=torch.float32, device=cuda_device)
    for e in range(256):
        b, s = synth.make_weight(7168, 2048, "normal", g2, cuda_device)
        B2[e] = b
        sb2[e] = s
    D2 = synth.sentinel_output((Mt, 7168), cuda_device)
    fg.fp8_grouped_gemm_nt_contiguous(A2, sa2, B2, sb2, D2, mi)
    torch.cuda.synchronize()
    D2v = D2.view(torch.int16)
    assert bool((D2v[pad] == -1).all()) and not bool((D2v[~pad] == -1).any())
    A2h, sa2h = A2.cpu().numpy(), sa2.cpu().numpy()
    ref2 = []
    for r in rows:
        e = int(mih[r])
        b, _ = oracle.gemm_nt_sampled(A2h, sa2h, B2[e].cpu().numpy(), sb2[e].cpu().numpy(), [r], np.arange(7168))
        ref2.append(b[0])
    compare("normal", bits_of(D2)[rows], np.stack(ref2), "moe down")


@pytest.mark.parametrize("G", [1024, 777])
def test_masked_maximum_group_count(cuda_device, G):
    # the largest group count the masked call accepts (the live-tile prefix sum over
    # every group is built in LDS) and a ragged one; masked_m spans empty, partial and
    # full groups
    M_max, N, K = 32, 256, 256
    rng = np.random.default_rng(G)
    mm = rng.integers(0, M_max + 1, G)
    mm[:3] = [0, M_max, 1]
    c = synth.masked_case(G, M_max, N, K, seed=G, device=cuda_device, masked_m=mm.tolist(), expected_m=16)
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm.tolist(), d_bits(c))
    for tile in (None, (64, 64, 1), (128, 128, 1)):
        got = bits_of(run_masked(c, tile))
        live = np.arange(M_max)[None, :] < mm[:, None]
        assert np.all(got[~live] == SENT), f"dead rows written (G={G}, {tile})"
        compare("normal", got[live], ref[live], f"masked G={G} {tile}")


def test_masked_rejects_too_many_groups():
    # the masked call's host check: more groups than the device prefix sum holds
    import ctypes
    P = ctypes.c_void_p
    st = fg.lib().fp8_grouped_gemm_nt_masked(P(1 << 20), 256, P(1 << 20), 32, P(1 << 20), 256, P(1 << 20),
                                             P(1 << 20), 256, P(1 << 20), 1025, 32, 256, 256, 16, None, 0, None)
    assert st == -2


@pytest.mark.parametrize("tile", [(64, 64, 2), (128, 128, 4), (256, 128, 3), (128, 256, 2), (64, 128, 8), (128, 64, 5),
                                  (128, 96, 3)],
                         ids=lambda t: "%dx%d_s%d" % t)
@pytest.mark.parametrize("kind", ["normal", "e1", "e1-ue8m0"])
def test_masked_split_k_forced(cuda_device, tile, kind):
    """Masked calls split K too (a K slice per unit, partials reduced by the last arrival
    into the live tile's workspace slot): empty, partial and full groups."""
    mm = [0, 300, 512, 1]
    ue = kind.endswith("ue8m0")
    kind = kind.split("-")[0]
    c = synth.masked_case(4, 512, 384, 1152, seed=9100 + tile[0] + tile[2], device=cuda_device, masked_m=mm,
                          expected_m=256, kind=kind)
    nbytes = forced_workspace_bytes(fg.KIND_MASKED, 512, 384, 1152, 4, tile)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=cuda_device)
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm, d_bits(c))
    for call in range(2):   # the workspace is reused
        D = c["D"].clone()
        with fg.force_config(*tile):
            fg.fp8_grouped_gemm_nt_masked(c["A"], c["sa"], c["B"], c["sb"], D, c["masked_m"], 256, ws, ue8m0=ue)
        torch.cuda.synchronize()
        got = bits_of(D)
        for g, live in enumerate(mm):
            assert np.all(got[g, live:] == SENT), f"dead rows of group {g} written"
            compare(kind, got[g, :live], ref[g, :live], f"masked split {tile} ue8m0={ue} group {g} call {call}")
        assert int(ws[:16384].count_nonzero()) == 0, "split-K counters must be left at zero"


def test_masked_split_k_falls_back_when_live_tiles_exceed_the_workspace(cuda_device):
    """The workspace is sized for twice expected_m rows per group; a call whose groups hold
    more live tiles than that runs unsplit on the device, with the same results."""
    mm = [500, 512, 450]
    c = synth.masked_case(3, 512, 256, 1024, seed=9200, device=cuda_device, masked_m=mm, expected_m=32)
    tile = (64, 64, 4)
    with fg.force_config(*tile):
        small = fg.workspace_size(fg.KIND_MASKED, 512, 256, 1024, 3, 32)   # capacity: 64 rows per group
    assert small > 16384
    ws = torch.zeros(small, dtype=torch.uint8, device=cuda_device)
    D = c["D"].clone()
    with fg.force_config(*tile):
        fg.fp8_grouped_gemm_nt_masked(c["A"], c["sa"], c["B"], c["sb"], D, c["masked_m"], 32, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm, d_bits(c))
    got = bits_of(D)
    for g, live in enumerate(mm):
        assert np.all(got[g, live:] == SENT)
        compare("normal", got[g, :live], ref[g, :live], f"fallback group {g}")
    assert int(ws[:16384].count_nonzero()) == 0
