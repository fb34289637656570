"""GPU parity: the HIP library against the CPU oracle, element by element.

Inputs are seeded (long_context_compressed_csa_amd.synth) and identical on
both sides (bf16 values are upcast exactly for the oracle).  Each test prints
the case it runs before touching the GPU.
"""

import math
import sys

import numpy as np
import pytest
import torch

import long_context_compressed_csa_amd as L
from long_context_compressed_csa_amd import synth
import oracle as O
from parity_helpers import assert_close, assert_index_sets, bf16_ulp, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    L.load_library()
    yield
    torch.cuda.synchronize()


def g(t):
    return t.to(DEV).contiguous()


# ------------------------------------------------------------- compressor --

@pytest.mark.parametrize("dtype,n,c,m,b", [
    (torch.float32, 64, 32, 4, 1),        # tiny layer, fixed m=4 kernel
    (torch.float32, 70, 36, 4, 2),        # ragged tail, c % 4 == 0
    (torch.float32, 45, 7, 4, 1),         # c not a multiple of the vector width
    (torch.bfloat16, 1027, 512, 4, 2),    # several entries per workgroup + ragged tail
    (torch.float32, 99, 24, 3, 1),        # other ratio: generic kernel
    (torch.bfloat16, 260, 128, 16, 1),    # generic kernel, row split over parts
])
def test_compress_overlap(dtype, n, c, m, b):
    say(f"compress overlap dtype={dtype} n={n} c={c} m={m} b={b}")
    d = synth.compress_inputs(True, n=n, c=c, m=m, dtype=dtype, seed=11, b=b)
    out = L.csa_compress(*(g(d[k]) for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    torch.cuda.synchronize()
    for s in range(b):
        want = O.compress_overlap(*(to64(d[k][s]) for k in ("Ca", "Cb", "Za", "Zb")),
                                  to64(d["Ba"]), to64(d["Bb"]), m)
        assert_close(out[s], want, dtype, f"seq {s}")


@pytest.mark.parametrize("dtype,n,c,mp,b", [
    (torch.bfloat16, 2048 + 77, 512, 128, 1),
    (torch.float32, 300, 20, 8, 2),
    (torch.bfloat16, 640, 512, 4, 1),
    (torch.float32, 1, 8, 1, 1),          # degenerate ratio 1: the entry is the row itself
    (torch.float32, 40 * 5 + 13, 24, 40, 2),   # one workgroup per entry: partial last round, few channels
    (torch.bfloat16, 64 * 3, 128, 64, 1),      # one workgroup per entry, c = 128
])
def test_compress_pool(dtype, n, c, mp, b):
    say(f"compress pool dtype={dtype} n={n} c={c} m'={mp} b={b}")
    d = synth.compress_inputs(False, n=n, c=c, m=mp, dtype=dtype, seed=12, b=b)
    out = L.csa_compress(g(d["C"]), None, g(d["Z"]), None, g(d["B"]), None, mp, overlap=False)
    torch.cuda.synchronize()
    for s in range(b):
        want = O.compress_pool(to64(d["C"][s]), to64(d["Z"][s]), to64(d["B"]), mp)
        assert_close(out[s], want, dtype, f"seq {s}")
    if mp == 1:
        assert torch.equal(out.cpu(), d["C"][:, : n].to(out.dtype))


def test_compress_overlap_grid_stride_channel_reload():
    # more (entry, channel) units than the grid has threads, with a channel
    # count (9) that does not divide the grid stride: threads loop over
    # several units and change channel between them
    say("compress overlap grid-stride, 9 channels")
    n, c, m = 4 * 120_000, 36, 4
    d = synth.compress_inputs(True, n=n, c=c, m=m, dtype=torch.float32, seed=14)
    out = L.csa_compress(*(g(d[k]) for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    torch.cuda.synchronize()
    want = O.compress_overlap(*(to64(d[k][0]) for k in ("Ca", "Cb", "Za", "Zb")), to64(d["Ba"]), to64(d["Bb"]), m)
    assert_close(out[0], want, torch.float32, "grid stride")


def test_compress_continues_from_previous_block_state():
    say("compress with previous-block state")
    d = synth.compress_inputs(True, n=64, c=512, m=4, dtype=torch.bfloat16, seed=13, b=2)
    cut = 24
    pcb, pzb = g(d["Cb"][:, cut - 4:cut]), g(d["Zb"][:, cut - 4:cut])
    tail = L.csa_compress(*(g(d[k][:, cut:]) for k in ("Ca", "Cb", "Za", "Zb")), g(d["Ba"]), g(d["Bb"]),
                          4, prev_Cb=pcb, prev_Zb=pzb)
    torch.cuda.synchronize()
    for s in range(2):
        want = O.compress_overlap(*(to64(d[k][s]) for k in ("Ca", "Cb", "Za", "Zb")),
                                  to64(d["Ba"]), to64(d["Bb"]), 4)[cut // 4:]
        assert_close(tail[s], want, torch.bfloat16, f"seq {s}")


def test_compress_full_size_sweep():
    # n = 65536, c = 512, both forms, every output element
    for overlap in (True, False):
        say(f"compress full size overlap={overlap}")
        d = synth.compress_inputs(overlap, seed=2)
        if overlap:
            out = L.csa_compress(*(g(d[k]) for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), 4)
            want = O.compress_overlap(*(to64(d[k][0]) for k in ("Ca", "Cb", "Za", "Zb")),
                                      to64(d["Ba"]), to64(d["Bb"]), 4)
        else:
            out = L.csa_compress(g(d["C"]), None, g(d["Z"]), None, g(d["B"]), None, 128, overlap=False)
            want = O.compress_pool(to64(d["C"][0]), to64(d["Z"][0]), to64(d["B"]), 128)
        torch.cuda.synchronize()
        assert_close(out[0], want, torch.bfloat16, f"overlap={overlap}")


def test_compress_weights_sum_to_one_on_gpu():
    # constant values C = 1 make the output the sum of the weights
    say("compress sum of weights")
    d = synth.compress_inputs(True, n=256, c=64, m=4, dtype=torch.float32, seed=14)
    ones = torch.ones_like(d["Ca"])
    out = L.csa_compress(g(ones), g(ones), g(d["Za"]), g(d["Zb"]), g(d["Ba"]), g(d["Bb"]), 4)
    torch.cuda.synchronize()
    assert float((out.cpu().double() - 1).abs().max()) < 1e-6


# ---------------------------------------------------------------- indexer --

def _oracle_index(qI, w, KI, t_pos, m, k):
    sc = O.index_scores(to64(qI), to64(w), to64(KI), t_pos, m)
    n_comp = KI.shape[0]
    vis = np.array([min((int(t) + 1) // m, n_comp) for t in t_pos])
    idx = np.stack([O.topk_select(sc[r], vis[r], k) for r in range(len(t_pos))])
    return idx, sc, vis


def test_index_topk_tiny_fp32():
    say("index tiny fp32")
    d = synth.tiny_inputs()
    p = d["params"]
    idx, sc = L.csa_index_topk(g(d["qI"]), g(d["w"]), g(d["KIcomp"]), 0, p["m"], p["k"], score=True)
    torch.cuda.synchronize()
    want, osc, vis = _oracle_index(d["qI"], d["w"], d["KIcomp"], np.arange(p["n"]), p["m"], p["k"])
    assert_index_sets(idx[0].cpu().numpy(), want, osc, vis, p["k"])
    # scores of the selected entries
    gi = idx[0].cpu().numpy()
    for r in range(p["n"]):
        for j, s in enumerate(gi[r]):
            if s >= 0:
                assert abs(float(sc[0, r, j]) - osc[r, s]) <= 1e-4 * max(1.0, abs(osc[r, s]))


@pytest.mark.parametrize("n_q,t0,nh,cI,k,b", [
    (301, 0, 64, 128, 16, 1),      # MFMA, 4 queries per workgroup, ragged query tail
    (37, 1000, 32, 64, 40, 2),     # other head / dim counts, t0 > 0, batch 2
    (3, 7000, 64, 128, 100, 2),    # few queries: keys split over workgroups
])
def test_index_topk_bf16_mfma(n_q, t0, nh, cI, k, b):
    say(f"index bf16 n_q={n_q} t0={t0} nh={nh} cI={cI} k={k} b={b}")
    m = 4
    n_comp = (t0 + n_q) // m
    gen = torch.Generator().manual_seed(21)
    qI = torch.randn((b, n_q, nh, cI), generator=gen).to(torch.bfloat16)
    KI = torch.randn((b, n_comp, cI), generator=gen).to(torch.bfloat16)
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    idx, sc = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k, score=True)
    torch.cuda.synchronize()
    t_pos = np.arange(t0, t0 + n_q)
    for s in range(b):
        want, osc, vis = _oracle_index(qI[s], w[s], KI[s], t_pos, m, k)
        nt = assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        gi, gs = idx[s].cpu().numpy(), sc[s].cpu().double().numpy()
        sel = gi >= 0
        rows = np.nonzero(sel)
        ref = osc[rows[0], gi[sel]]
        assert np.max(np.abs(gs[sel] - ref)) <= 1e-4 * max(1.0, np.abs(ref).max())
        say(f"  seq {s}: near-ties decided differently: {nt}")


def test_index_topk_negative_weights_and_multistage():
    # negative head weights give negative scores; 20000 candidates need the
    # multi-stage selection (chunks of 4096)
    say("index multistage, negative weights")
    m, k, b, n_comp = 4, 512, 2, 20000
    t0 = n_comp * m - 1
    gen = torch.Generator().manual_seed(22)
    qI = torch.randn((b, 1, 64, 128), generator=gen).to(torch.bfloat16)
    KI = torch.randn((b, n_comp, 128), generator=gen).to(torch.bfloat16)
    w = torch.randn((b, 1, 64), generator=gen)
    idx, sc = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in range(b):
        want, osc, vis = _oracle_index(qI[s], w[s], KI[s], [t0], m, k)
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        assert float(osc.min()) < 0       # the candidate list does hold negative scores


def test_index_topk_exact_ties_lower_index_wins():
    # identical keys give identical scores: the lowest indices must be taken
    say("index exact ties")
    m, k, n_q = 1, 5, 2
    n_comp = 40
    KI = torch.ones((n_comp, 128), dtype=torch.bfloat16)
    KI[7] = 2.0                                     # one strictly larger entry
    qI = torch.ones((n_q, 64, 128), dtype=torch.bfloat16)
    w = torch.ones((n_q, 64))
    t0 = n_comp - 1
    idx = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k)
    torch.cuda.synchronize()
    got = idx[0].cpu().numpy()
    assert got[0].tolist() == [0, 1, 2, 3, 7]
    assert got[1].tolist() == [0, 1, 2, 3, 7]


@pytest.mark.parametrize("n_comp,k,bump", [
    (5000, 100, [4999, 123, 2048]),   # ties across three segments, a few strictly larger entries
    (20480, 1000, [7]),               # every segment keeps 1000 ties: the merge takes two chunks
])
def test_index_topk_long_lists_exact_ties(n_comp, k, bump):
    # equal scores everywhere except a few larger entries: the lower indices
    # must win the ties, however the candidate list is split
    say(f"index long-list ties n_comp={n_comp} k={k}")
    m = 1
    KI = torch.ones((n_comp, 128), dtype=torch.bfloat16)
    for e in bump:
        KI[e] = 2.0
    qI = torch.ones((1, 64, 128), dtype=torch.bfloat16)
    w = torch.ones((1, 64))
    idx = L.csa_index_topk(g(qI), g(w), g(KI), n_comp - 1, m, k)
    torch.cuda.synchronize()
    want, _, _ = _oracle_index(qI, w, KI, [n_comp - 1], m, k)
    assert want[0].tolist() == sorted(bump + [e for e in range(n_comp) if e not in bump][: k - len(bump)])
    assert idx[0, 0].cpu().numpy().tolist() == want[0].tolist()


@pytest.mark.parametrize("n_distinct,k", [(1, 300), (3, 700), (17, 512)])
def test_index_topk_fused_selection_ties(n_distinct, k):
    # four or more queries whose lists fit one segment select inside the
    # scoring kernel: keys drawn from a few distinct rows make long runs of
    # exactly equal scores around the k-th, which the lower indices must win
    say(f"index fused selection ties n_distinct={n_distinct} k={k}")
    m, n_q, n_comp = 1, 9, 2048
    t0 = n_comp - n_q
    gen = torch.Generator().manual_seed(25)
    rows = torch.randn((n_distinct, 128), generator=gen)
    KI = rows[torch.randint(0, n_distinct, (n_comp,), generator=gen)].to(torch.bfloat16)
    qI = torch.randn((n_q, 64, 128), generator=gen).to(torch.bfloat16)
    w = torch.nn.functional.softplus(torch.randn((n_q, 64), generator=gen))
    idx = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k)
    torch.cuda.synchronize()
    want, osc, vis = _oracle_index(qI, w, KI, np.arange(t0, t0 + n_q), m, k)
    # equal keys give bit-equal scores on both sides, so the sets must agree exactly
    assert np.array_equal(idx[0].cpu().numpy(), want)


def test_index_topk_fused_nothing_visible():
    # no entry is complete for any query: every index is padding
    say("index fused, no visible entries")
    m, n_q, k = 8, 4, 16
    qI = torch.randn((n_q, 64, 128)).to(torch.bfloat16)
    KI = torch.zeros((1, 128), dtype=torch.bfloat16)
    w = torch.ones((n_q, 64))
    idx = L.csa_index_topk(g(qI), g(w), g(KI), 0, m, k, n_comp=0)
    torch.cuda.synchronize()
    assert (idx.cpu() == -1).all()


def _fp8_oracle_index(qI8, w, KI8, t_pos, m, k):
    # the oracle scores the values the codes stand for
    dq = O.fp8_e4m3_decode(qI8.view(torch.uint8).numpy())
    dk = O.fp8_e4m3_decode(KI8.view(torch.uint8).numpy())
    sc = O.index_scores(dq, to64(w), dk, t_pos, m)
    n_comp = KI8.shape[0]
    vis = np.array([min((int(t) + 1) // m, n_comp) for t in t_pos])
    idx = np.stack([O.topk_select(sc[r], vis[r], k) for r in range(len(t_pos))])
    return idx, sc, vis


@pytest.mark.parametrize("b,n_q,n_comp,k,nh,cI", [
    (2, 1, 20000, 512, 64, 128),    # streaming FP8 scorer, threshold selection
    (2, 3, 1500, 100, 64, 128),     # streaming FP8 scorer, one segment per row, rows of different length
    (1, 2, 9000, 300, 32, 64),      # other head / dimension counts
    (1, 6, 1200, 64, 64, 128),      # four or more queries: block-scaled MFMA with fused selection
    (2, 37, 1500, 300, 32, 128),    # fused, 32 heads, a partial last query block
    (1, 5, 600, 40, 128, 128),      # fused, 128 heads
    (1, 9, 3000, 100, 64, 128),     # lists longer than one workgroup: MFMA scores + general selection
    (1, 6, 700, 40, 48, 64),        # shape without an MFMA kernel: generic scoring
    (1, 2, 700, 40, 48, 40),        # the same with few queries
])
def test_index_topk_fp8(b, n_q, n_comp, k, nh, cI):
    # E4M3 indexer queries and keys: the same selection as the oracle's over
    # the decoded values, apart from near ties
    say(f"index fp8 b={b} n_q={n_q} n_comp={n_comp} k={k} nh={nh} cI={cI}")
    m = 4
    t0 = n_comp * m - n_q
    gen = torch.Generator().manual_seed(26)
    qI = synth.to_fp8(torch.randn((b, n_q, nh, cI), generator=gen) / math.sqrt(cI))
    KI = synth.to_fp8(torch.randn((b, n_comp, cI), generator=gen) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    idx, sc = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in range(b):
        want, osc, vis = _fp8_oracle_index(qI[s], w[s], KI[s], np.arange(t0, t0 + n_q), m, k)
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        gi, gs = idx[s].cpu().numpy(), sc[s].cpu().double().numpy()
        sel = gi >= 0
        ref = osc[np.nonzero(sel)[0], gi[sel]]
        assert np.max(np.abs(gs[sel] - ref)) <= 1e-3 * max(1.0, np.abs(ref).max())


def test_index_topk_fp8_prefill_full_size_sampled():
    # the CSA prefill shape (n = 8192, 2048 entries, 64 x 128 indexer, k =
    # 512) with E4M3 codes, the keys in a cache with spare rows: fused MFMA
    # scorer, sampled queries
    say("index fp8 prefill n=8192 (sampled queries)")
    d = synth.prefill_inputs()
    p = d["params"]
    qI = synth.to_fp8(d["qI"])
    KI = synth.to_fp8(torch.cat([d["KIcomp"].float(), torch.randn((40, d["KIcomp"].shape[1]))]))
    ne = d["KIcomp"].shape[0]
    idx = L.csa_index_topk(g(qI), g(d["w"]), g(KI), 0, p["m"], p["k"], n_comp=ne)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(2040, 2056), np.arange(8184, 8192),
                                     np.random.default_rng(3).integers(0, 8192, 40)]))
    want, osc, vis = _fp8_oracle_index(qI[rows], d["w"][rows], KI[:ne], rows, p["m"], p["k"])
    nt = assert_index_sets(idx[0, rows].cpu().numpy(), want, osc, vis, p["k"])
    say(f"  sampled {len(rows)} queries, near-ties: {nt}")


def test_index_topk_fp8_one_million_context_sampled():
    # the 1M-token decode shape (8 sequences x 262144 entries, one query
    # each, 64 x 128 indexer, k = 512) with E4M3 codes: the launch the
    # decode step makes, checked on two sequences
    say("index fp8 8 x 262144 entries (sampled sequences)")
    b, n_comp, nh, cI, m, k = 8, 262144, 64, 128, 4, 512
    gen = torch.Generator(device=DEV).manual_seed(29)
    KI = synth.to_fp8(torch.randn((b, n_comp, cI), generator=gen, device=DEV) / math.sqrt(cI))
    qI = synth.to_fp8(torch.randn((b, 1, nh, cI), generator=gen, device=DEV) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, 1, nh), generator=gen, device=DEV))
    t0 = n_comp * m - 1
    idx, sc = L.csa_index_topk(qI, w, KI, t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in (0, b - 1):
        want, osc, vis = _fp8_oracle_index(qI[s].cpu(), w[s].cpu(), KI[s].cpu(), np.array([t0]), m, k)
        assert vis[0] == n_comp
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        gi, gs = idx[s, 0].cpu().numpy(), sc[s, 0].cpu().double().numpy()
        ref = osc[0, gi]
        assert np.max(np.abs(gs - ref)) <= 1e-3 * max(1.0, np.abs(ref).max())


def _mx_oracle_index(qc, qs, w, kc, ks, t_pos, m, k):
    # the oracle scores the values the MXFP4 codes stand for
    dq = O.mxfp4_decode(qc.numpy(), qs.numpy())
    dk = O.mxfp4_decode(kc.numpy(), ks.numpy())
    sc = O.index_scores(dq, to64(w), dk, t_pos, m)
    n_comp = kc.shape[0]
    vis = np.array([min((int(t) + 1) // m, n_comp) for t in t_pos])
    idx = np.stack([O.topk_select(sc[r], vis[r], k) for r in range(len(t_pos))])
    return idx, sc, vis


@pytest.mark.parametrize("b,n_q,n_comp,k,nh,cI", [
    (2, 1, 20000, 512, 64, 128),    # streaming MXFP4 scorer, threshold selection
    (2, 3, 1500, 100, 64, 128),     # streaming, one segment per row, rows of different length
    (1, 2, 9000, 300, 32, 128),     # 32 heads
    (1, 1, 5000, 200, 128, 128),    # 128 heads
    (1, 6, 1200, 64, 64, 128),      # four or more queries: MFMA scorer with fused selection
    (2, 37, 1500, 300, 32, 128),    # fused, 32 heads, a partial last query block
    (1, 5, 600, 40, 128, 128),      # fused, 128 heads
    (1, 9, 3000, 100, 64, 128),     # lists longer than one workgroup: MFMA scores + general selection
    (1, 6, 1200, 64, 48, 64),       # no MFMA kernel for this shape: generic scoring
    (1, 2, 700, 40, 48, 64),        # the same with few queries
])
def test_index_topk_mxfp4(b, n_q, n_comp, k, nh, cI):
    # MXFP4 indexer queries and keys: the same selection as the oracle's over
    # the decoded values, apart from near ties
    say(f"index mxfp4 b={b} n_q={n_q} n_comp={n_comp} k={k} nh={nh} cI={cI}")
    m = 4
    t0 = n_comp * m - n_q
    gen = torch.Generator().manual_seed(31)
    qc, qs = synth.to_mxfp4(torch.randn((b, n_q, nh, cI), generator=gen) / math.sqrt(cI))
    kc, ks = synth.to_mxfp4(torch.randn((b, n_comp, cI), generator=gen) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    idx, sc = L.csa_index_topk_mxfp4(g(qc), g(qs), g(w), g(kc), g(ks), t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in range(b):
        want, osc, vis = _mx_oracle_index(qc[s], qs[s], w[s], kc[s], ks[s], np.arange(t0, t0 + n_q), m, k)
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        gi, gs = idx[s].cpu().numpy(), sc[s].cpu().double().numpy()
        sel = gi >= 0
        ref = osc[np.nonzero(sel)[0], gi[sel]]
        assert np.max(np.abs(gs[sel] - ref)) <= 1e-4 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("n_q", [1, 6])
def test_index_topk_mxfp4_keys_in_a_larger_cache(n_q):
    # keys in a cache with spare rows (the per-sequence stride is the cache's
    # capacity, not n_comp), for the streaming and the four-query scorer
    say(f"index mxfp4 cache with spare rows n_q={n_q}")
    b, n_comp, cap, nh, cI, m, k = 2, 3000, 3100, 64, 128, 4, 200
    gen = torch.Generator().manual_seed(59)
    qc, qs = synth.to_mxfp4(torch.randn((b, n_q, nh, cI), generator=gen) / math.sqrt(cI))
    kc, ks = synth.to_mxfp4(torch.randn((b, cap, cI), generator=gen) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    t0 = n_comp * m - n_q
    idx, sc = L.csa_index_topk_mxfp4(g(qc), g(qs), g(w), g(kc), g(ks), t0, m, k, n_comp=n_comp, score=True)
    torch.cuda.synchronize()
    for s in range(b):
        want, osc, vis = _mx_oracle_index(qc[s], qs[s], w[s], kc[s, :n_comp], ks[s, :n_comp],
                                          np.arange(t0, t0 + n_q), m, k)
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")


def test_index_topk_mxfp4_one_million_context_sampled():
    # the 1M-token decode shape with MXFP4 codes (Gaussian keys and queries
    # quantised on the GPU): the launch the decode step makes, checked on two
    # sequences
    say("index mxfp4 8 x 262144 entries (sampled sequences)")
    b, n_comp, nh, cI, m, k = 8, 262144, 64, 128, 4, 512
    gen = torch.Generator(device=DEV).manual_seed(37)
    kc, ks = synth.to_mxfp4(torch.randn((b, n_comp, cI), generator=gen, device=DEV) / math.sqrt(cI))
    qc, qs = synth.to_mxfp4(torch.randn((b, 1, nh, cI), generator=gen, device=DEV) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, 1, nh), generator=gen, device=DEV))
    t0 = n_comp * m - 1
    idx, sc = L.csa_index_topk_mxfp4(qc, qs, w, kc, ks, t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in (0, b - 1):
        want, osc, vis = _mx_oracle_index(qc[s].cpu(), qs[s].cpu(), w[s].cpu(), kc[s].cpu(), ks[s].cpu(),
                                          np.array([t0]), m, k)
        assert vis[0] == n_comp
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")
        gi, gs = idx[s, 0].cpu().numpy(), sc[s, 0].cpu().double().numpy()
        ref = osc[0, gi]
        assert np.max(np.abs(gs - ref)) <= 1e-4 * max(1.0, np.abs(ref).max())


def test_index_topk_mxfp4_prefill_full_size_sampled():
    # the CSA prefill shape (n = 8192, 2048 entries, 64 x 128 indexer, k =
    # 512) with MXFP4 codes: fused MFMA scorer, sampled queries
    say("index mxfp4 prefill n=8192 (sampled queries)")
    d = synth.prefill_inputs()
    p = d["params"]
    qc, qs = synth.to_mxfp4(d["qI"].float())
    kc, ks = synth.to_mxfp4(d["KIcomp"].float())
    idx, sc = L.csa_index_topk_mxfp4(g(qc), g(qs), g(d["w"]), g(kc), g(ks), 0, p["m"], p["k"], score=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(2040, 2056), np.arange(8184, 8192),
                                     np.random.default_rng(1).integers(0, 8192, 40)]))
    want, osc, vis = _mx_oracle_index(qc[rows], qs[rows], d["w"][rows], kc, ks, rows, p["m"], p["k"])
    nt = assert_index_sets(idx[0, rows].cpu().numpy(), want, osc, vis, p["k"])
    say(f"  sampled {len(rows)} queries, near-ties: {nt}")


def test_index_topk_mxfp4_matches_decoded_fp32_path():
    # the same codes through the float32 entry point (decoded on the host):
    # identical selection, scores within float32 summation-order error
    say("index mxfp4 vs decoded float32")
    b, n_q, n_comp, nh, cI, m, k = 2, 1, 12000, 64, 128, 4, 256
    gen = torch.Generator().manual_seed(41)
    qc, qs = synth.to_mxfp4(torch.randn((b, n_q, nh, cI), generator=gen) / math.sqrt(cI))
    kc, ks = synth.to_mxfp4(torch.randn((b, n_comp, cI), generator=gen) / math.sqrt(cI))
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    t0 = n_comp * m - 1
    dq = torch.from_numpy(O.mxfp4_decode(qc.numpy(), qs.numpy())).float()
    dk = torch.from_numpy(O.mxfp4_decode(kc.numpy(), ks.numpy())).float()
    i1, s1 = L.csa_index_topk_mxfp4(g(qc), g(qs), g(w), g(kc), g(ks), t0, m, k, score=True)
    i2, s2 = L.csa_index_topk(g(dq), g(w), g(dk), t0, m, k, score=True)
    torch.cuda.synchronize()
    for s in range(b):
        a1, a2 = set(i1[s, 0].cpu().tolist()), set(i2[s, 0].cpu().tolist())
        assert len(a1 ^ a2) <= 4, len(a1 ^ a2)   # near-ties only
        if a1 == a2:
            assert torch.allclose(s1[s], s2[s], rtol=1e-5, atol=1e-6)


def _mx_edge_rows(gen, c):
    # Gaussian rows at several magnitudes plus blocks that hit every rule:
    # all zero, values on each E2M1 midpoint of their block scale, saturation,
    # negative zero-rounding, tiny (subnormal range) and large magnitudes
    x = torch.randn((12, c), generator=gen) * torch.exp2(torch.randint(-30, 30, (12, 1), generator=gen).float())
    x[0, :32] = 0.0
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9])
    x[1, :32] = torch.cat([torch.tensor([4.0]), mids, -mids, torch.zeros(15)]) * 2.0 ** -5
    x[2, :32] = torch.linspace(-7.99, 7.99, 32) * 2.0 ** 40
    x[3, :32] = torch.cat([torch.tensor([1.0]), -torch.full((31,), 0.01)])
    x[4, :32] = torch.randn(32, generator=gen) * 2.0 ** -130
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_mxfp4_bit_exact(dtype):
    # codes and scales byte for byte against the oracle's encoder of the same values
    say(f"quantize mxfp4 {dtype}")
    gen = torch.Generator().manual_seed(43)
    for c in (32, 128, 512):
        x = _mx_edge_rows(gen, c).to(dtype)
        codes, scales = L.csa_quantize_mxfp4(g(x))
        torch.cuda.synchronize()
        wc, wsc = O.mxfp4_encode(to64(x))
        assert np.array_equal(scales.cpu().numpy(), wsc), f"c={c} scales"
        assert np.array_equal(codes.cpu().numpy(), wc), f"c={c} codes"
    # a large batch: every row Gaussian at its own magnitude
    x = (torch.randn((4096, 128), generator=gen) * torch.exp2(torch.randint(-8, 8, (4096, 1), generator=gen).float()))
    x = x.to(dtype)
    codes, scales = L.csa_quantize_mxfp4(g(x))
    torch.cuda.synchronize()
    wc, wsc = O.mxfp4_encode(to64(x))
    assert np.array_equal(scales.cpu().numpy(), wsc) and np.array_equal(codes.cpu().numpy(), wc)


def test_quantize_mxfp4_appends_rows_in_place():
    # one row per sequence written at entry e of [b, cap, ...] caches through
    # the batch strides, the rest of the caches untouched (the decode append)
    say("quantize mxfp4 in-place append")
    lib = L.load_library()
    b, cap, c, e = 3, 10, 128, 7
    gen = torch.Generator().manual_seed(47)
    src = g(torch.randn((b, cap, c), generator=gen).to(torch.bfloat16))
    codes = torch.full((b, cap, c // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((b, cap, c // 32), 0xA5, dtype=torch.uint8, device=DEV)
    rc = lib.csa_quantize_mxfp4(src[:, e].data_ptr(), cap * c, b, c, 1, codes[:, e].data_ptr(), cap * c // 2,
                                scales[:, e].data_ptr(), cap * c // 32, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    wc, wsc = O.mxfp4_encode(to64(src[:, e].cpu()))
    assert np.array_equal(codes[:, e].cpu().numpy(), wc) and np.array_equal(scales[:, e].cpu().numpy(), wsc)
    rest = [i for i in range(cap) if i != e]
    assert (codes[:, rest] == 0x5A).all() and (scales[:, rest] == 0xA5).all()


def test_index_topk_long_lists_rows_differ():
    # few queries whose visible counts differ (4095, 4095, 4096 entries)
    say("index long lists, rows with different visibility")
    m, k, n_q, t0, n_comp = 4, 300, 3, 16381, 4096
    gen = torch.Generator().manual_seed(23)
    qI = torch.randn((1, n_q, 64, 128), generator=gen).to(torch.bfloat16)
    KI = torch.randn((1, n_comp, 128), generator=gen).to(torch.bfloat16)
    w = torch.nn.functional.softplus(torch.randn((1, n_q, 64), generator=gen))
    idx, sc = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k, score=True)
    torch.cuda.synchronize()
    want, osc, vis = _oracle_index(qI[0], w[0], KI[0], np.arange(t0, t0 + n_q), m, k)
    assert list(vis) == [4095, 4095, 4096]
    assert_index_sets(idx[0].cpu().numpy(), want, osc, vis, k, "rows")


@pytest.mark.parametrize("dtype,n_q", [(torch.bfloat16, 5), (torch.float32, 2)])
def test_index_topk_long_lists_general_path(dtype, n_q):
    # more than 2048 candidates scored by the 4-query MFMA kernel or the
    # generic kernel: the multi-stage selection without group maxima
    say(f"index long lists general path dtype={dtype} n_q={n_q}")
    m, k, b = 4, 256, 2
    t0 = 12000
    n_comp = (t0 + n_q) // m
    gen = torch.Generator().manual_seed(24)
    qI = torch.randn((b, n_q, 64, 128), generator=gen).to(dtype)
    KI = torch.randn((b, n_comp, 128), generator=gen).to(dtype)
    w = torch.nn.functional.softplus(torch.randn((b, n_q, 64), generator=gen))
    idx = L.csa_index_topk(g(qI), g(w), g(KI), t0, m, k)
    torch.cuda.synchronize()
    for s in range(b):
        want, osc, vis = _oracle_index(qI[s], w[s], KI[s], np.arange(t0, t0 + n_q), m, k)
        assert_index_sets(idx[s].cpu().numpy(), want, osc, vis, k, f"seq {s}")


def test_index_topk_prefill_full_size_sampled():
    say("index prefill n=8192 (sampled queries)")
    d = synth.prefill_inputs()
    p = d["params"]
    idx, sc = L.csa_index_topk(g(d["qI"]), g(d["w"]), g(d["KIcomp"]), 0, p["m"], p["k"], score=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(2040, 2056), np.arange(8184, 8192),
                                     np.random.default_rng(0).integers(0, 8192, 40)]))
    want, osc, vis = _oracle_index(d["qI"][rows], d["w"][rows], d["KIcomp"], rows, p["m"], p["k"])
    nt = assert_index_sets(idx[0, rows].cpu().numpy(), want, osc, vis, p["k"])
    say(f"  sampled {len(rows)} queries, near-ties: {nt}")


# -------------------------------------------------------------- attention --

def _oracle_idx_for(KI, qI, w, t_pos, m, k):
    idx, _, _ = _oracle_index(qI, w, KI, t_pos, m, k)
    return idx


def test_attend_tiny_fp32():
    say("attend tiny fp32")
    d = synth.tiny_inputs()
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    Cc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    Cc32 = torch.tensor(Cc, dtype=torch.float32)
    idx = _oracle_idx_for(d["KIcomp"], d["qI"], d["w"], np.arange(n), m, k)
    out = L.csa_attend(g(d["q"]), g(Cc32), g(torch.tensor(idx, dtype=torch.int32)), g(d["kv_raw"]),
                       g(d["sink"]), 0, m, nw, d["scale"])
    torch.cuda.synchronize()
    want = O.csa_attend(to64(d["q"]), Cc32.double().numpy(), idx, to64(d["kv_raw"]), 0, to64(d["sink"]),
                        np.arange(n), nw, d["scale"], m)
    assert_close(out[0], want, torch.float32)


@pytest.mark.parametrize("n,k,nw,b,unscaled,nh", [
    (300, 32, 16, 1, True, 64),     # sharp softmax (N(0,1) data), ragged tiles
    (200, 64, 128, 2, False, 128),  # two head groups, batch 2
    (96, 8, 200, 1, True, 64),      # window longer than the sequence
])
def test_attend_bf16_mfma(n, k, nw, b, unscaled, nh):
    say(f"attend bf16 n={n} k={k} n_win={nw} b={b} unscaled={unscaled} n_h={nh}")
    m = 4
    ds = [synth.prefill_inputs(n=n, seed=31 + s, n_h=nh, k=k, unscaled=unscaled) for s in range(b)]
    q = torch.stack([d["q"] for d in ds])
    raw = torch.stack([d["kv_raw"] for d in ds])
    Ccs, idxs = [], []
    for d in ds:
        Cc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
        Ccs.append(torch.tensor(Cc, dtype=torch.float32).to(torch.bfloat16))
        idxs.append(torch.tensor(_oracle_idx_for(d["KIcomp"], d["qI"], d["w"], np.arange(n), m, k),
                                 dtype=torch.int32))
    sink = ds[0]["sink"]
    out = L.csa_attend(g(q), g(torch.stack(Ccs)), g(torch.stack(idxs)), g(raw), g(sink), 0, m, nw,
                       ds[0]["scale"])
    torch.cuda.synchronize()
    for s in range(b):
        want = O.csa_attend(to64(q[s]), to64(Ccs[s]), idxs[s].numpy(), to64(raw[s]), 0, to64(sink),
                            np.arange(n), nw, ds[0]["scale"], m)
        assert_close(out[s], want, torch.bfloat16, f"seq {s}")


def test_attend_decode_split_and_invalid_indices():
    # one query per sequence: entries split over workgroups and merged;
    # idx holds padding, out-of-range and future indices that must be skipped
    say("attend decode split")
    m, k, nw, b, n_comp = 4, 96, 128, 2, 500
    t = n_comp * m + 2
    gen = torch.Generator().manual_seed(41)
    q = (torch.randn((b, 1, 64, 512), generator=gen)).to(torch.bfloat16)
    Cc = (torch.randn((b, n_comp + 10, 512), generator=gen)).to(torch.bfloat16)
    raw = (torch.randn((b, nw, 512), generator=gen)).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    idx = torch.stack([torch.sort(torch.randperm(n_comp, generator=gen)[:k]).values for _ in range(b)])
    idx = idx.to(torch.int32)[:, None, :]
    idx[:, 0, -3] = -1
    idx[:, 0, -2] = n_comp + 5          # exists in the buffer but is not complete yet
    idx[:, 0, -1] = 1 << 30
    raw_pos0 = t - nw + 1
    out = L.csa_attend(g(q), g(Cc), g(idx), g(raw), g(sink), t, m, nw, 1 / math.sqrt(512),
                       raw_pos0=raw_pos0, n_comp=n_comp)
    torch.cuda.synchronize()
    for s in range(b):
        i = idx[s].numpy()
        oidx = np.where((i >= 0) & (i < n_comp), i, -1)
        want = O.csa_attend(to64(q[s]), to64(Cc[s, :n_comp]), oidx, to64(raw[s]), raw_pos0, to64(sink), [t],
                            nw, 1 / math.sqrt(512), m)
        assert_close(out[s], want, torch.bfloat16, f"seq {s}")


def test_attend_decode_split_extreme_sinks():
    # the split merge's sink term at both ends: heads whose sink outweighs
    # every logit by e^40 (outputs near 0, each split's weight 2^-57 or
    # less), heads whose sink is negligible, the rest ordinary; CSA (5
    # splits per sequence) and HCA (32 splits) decode
    say("attend decode split, extreme sinks")
    gen = torch.Generator().manual_seed(44)
    sink = torch.randn(64, generator=gen)
    sink[:16] = 40.0
    sink[16:32] = -40.0
    scale = 1 / math.sqrt(512)
    m, k, nw, b, n_comp = 4, 96, 128, 2, 500
    t = n_comp * m + 2
    q = torch.randn((b, 1, 64, 512), generator=gen).to(torch.bfloat16)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    idx = torch.stack([torch.sort(torch.randperm(n_comp, generator=gen)[:k]).values for _ in range(b)])
    idx = idx.to(torch.int32)[:, None, :]
    raw_pos0 = t - nw + 1
    assert L.load_library().csa_attend_workspace_size(b, 1, t, n_comp, 64, 512, k, m, nw, 1) > 0
    out = L.csa_attend(g(q), g(Cc), g(idx), g(raw), g(sink), t, m, nw, scale, raw_pos0=raw_pos0)
    mp, nh_comp = 128, 2000
    th = nh_comp * mp + 5
    Ch = torch.randn((b, nh_comp, 512), generator=gen).to(torch.bfloat16)
    assert L.load_library().hca_attend_workspace_size(b, 1, th, nh_comp, 64, 512, mp, nw, 1) > 0
    outh = L.hca_attend(g(q), g(Ch), g(raw), g(sink), th, mp, nw, scale, raw_pos0=th - nw + 1)
    torch.cuda.synchronize()
    for s in range(b):
        want = O.csa_attend(to64(q[s]), to64(Cc[s]), idx[s].numpy(), to64(raw[s]), raw_pos0, to64(sink), [t], nw,
                            scale, m)
        assert_close(out[s], want, torch.bfloat16, f"csa seq {s}")
        wanth = O.hca_attend(to64(q[s]), to64(Ch[s]), to64(raw[s]), th - nw + 1, to64(sink), [th], mp, nw, scale)
        assert_close(outh[s], wanth, torch.bfloat16, f"hca seq {s}")
        assert np.abs(want[0, :16]).max() < 1e-10 and np.abs(wanth[0, :16]).max() < 1e-10


def test_attend_generic_bf16_small_heads():
    say("attend generic bf16")
    gen = torch.Generator().manual_seed(42)
    n, nh, c, m, k, nw = 40, 3, 48, 4, 3, 7
    q = torch.randn((n, nh, c), generator=gen).to(torch.bfloat16)
    Cc = torch.randn((n // m, c), generator=gen).to(torch.bfloat16)
    raw = torch.randn((n, c), generator=gen).to(torch.bfloat16)
    sink = torch.randn(nh, generator=gen)
    idx = np.stack([O.topk_select(np.random.default_rng(t).normal(size=n // m), (t + 1) // m, k)
                    for t in range(n)])
    out = L.csa_attend(g(q), g(Cc), g(torch.tensor(idx, dtype=torch.int32)), g(raw), g(sink), 0, m, nw, 0.2)
    torch.cuda.synchronize()
    want = O.csa_attend(to64(q), to64(Cc), idx, to64(raw), 0, to64(sink), np.arange(n), nw, 0.2, m)
    assert_close(out[0], want, torch.bfloat16)


def test_attend_prefill_full_size_sampled():
    say("attend prefill n=8192 (oracle indices, sampled queries)")
    d = synth.prefill_inputs()
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    Cc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    Cc16 = torch.tensor(Cc, dtype=torch.float32).to(torch.bfloat16)
    idx = _oracle_idx_for(d["KIcomp"], d["qI"], d["w"], np.arange(n), m, k)
    out = L.csa_attend(g(d["q"]), g(Cc16), g(torch.tensor(idx, dtype=torch.int32)), g(d["kv_raw"]),
                       g(d["sink"]), 0, m, nw, d["scale"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 6), [2047, 2048, 2051], np.arange(8188, 8192),
                                     np.random.default_rng(1).integers(0, n, 24)]))
    want = O.csa_attend(to64(d["q"][rows]), to64(Cc16), idx[rows], to64(d["kv_raw"]), 0, to64(d["sink"]),
                        rows, nw, d["scale"], m)
    assert_close(out[0, rows], want, torch.bfloat16)


def test_larger_model_shapes_prefill_sampled():
    # the pages' larger model's layer shapes (128 query heads, top-1024,
    # window 128, indexer 64 x 128, m = 4) at n = 8192: the library's
    # selection on sampled queries, and attention over blocks of queries
    # (oracle indices) at their positions
    say("larger model shapes: n_h=128, k=1024, n=8192 (sampled)")
    d = synth.prefill_inputs(n_h=128, k=1024)
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    assert (p["n_h"], k) == (128, 1024)
    idx, sc = L.csa_index_topk(g(d["qI"]), g(d["w"]), g(d["KIcomp"]), 0, m, k, score=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(4092, 4100), np.arange(8188, 8192),
                                     np.random.default_rng(2).integers(0, n, 16)]))
    want, osc, vis = _oracle_index(d["qI"][rows], d["w"][rows], d["KIcomp"], rows, m, k)
    assert_index_sets(idx[0, rows].cpu().numpy(), want, osc, vis, k)
    Cc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    Cc16 = torch.tensor(Cc, dtype=torch.float32).to(torch.bfloat16)
    for t0, nb in ((4090, 12), (8180, 12)):
        t_pos = np.arange(t0, t0 + nb)
        oi = _oracle_idx_for(d["KIcomp"], d["qI"][t0:t0 + nb], d["w"][t0:t0 + nb], t_pos, m, k)
        n_comp = min((t0 + nb) // m, Cc16.shape[0])
        out = L.csa_attend(g(d["q"][t0:t0 + nb]), g(Cc16), g(torch.tensor(oi, dtype=torch.int32)), g(d["kv_raw"]),
                           g(d["sink"]), t0, m, nw, d["scale"], n_comp=n_comp)
        torch.cuda.synchronize()
        w_out = O.csa_attend(to64(d["q"][t0:t0 + nb]), to64(Cc16), oi, to64(d["kv_raw"]), 0, to64(d["sink"]),
                             t_pos, nw, d["scale"], m)
        assert_close(out[0], w_out, torch.bfloat16, f"t0={t0}")


# -------------------------------------------------------------------- HCA --

@pytest.mark.parametrize("n,mp,nw,nh,dtype", [
    (700, 128, 128, 64, torch.bfloat16),
    (300, 16, 40, 64, torch.bfloat16),
    (64, 8, 16, 4, torch.float32),
])
def test_hca_layer_small(n, mp, nw, nh, dtype):
    say(f"hca layer n={n} m'={mp} n_win={nw} n_h={nh} {dtype}")
    d = synth.hca_inputs(n=n, seed=51, n_h=nh, m_prime=mp)
    if dtype == torch.float32:
        d = {k2: (v.float() if isinstance(v, torch.Tensor) and v.dtype == torch.bfloat16 else v)
             for k2, v in d.items()}
    Cc, out = L.hca_layer(g(d["C"]), g(d["Z"]), g(d["B"]), g(d["q"]), g(d["kv_raw"]), g(d["sink"]),
                          mp, nw, d["scale"])
    torch.cuda.synchronize()
    wCc, wout = O.hca_layer(to64(d["C"]), to64(d["Z"]), to64(d["B"]), to64(d["q"]), to64(d["kv_raw"]),
                            to64(d["sink"]), mp, nw, d["scale"])
    assert_close(Cc[0], wCc, dtype, "Ccomp")
    # the attention step reads entries stored in the storage dtype: the
    # oracle attends over its own entries rounded the same way
    Cc_in = torch.tensor(wCc, dtype=torch.float32).to(dtype)
    want = O.hca_attend(to64(d["q"]), to64(Cc_in), to64(d["kv_raw"]), 0, to64(d["sink"]), np.arange(n),
                        mp, nw, d["scale"])
    assert_close(out[0], want, dtype, "out")


def test_hca_attend_full_size_sampled():
    say("hca n=131072 (sampled queries)")
    d = synth.hca_inputs(device=DEV)
    p = d["params"]
    Cc, out = L.hca_layer(d["C"], d["Z"], d["B"], d["q"], d["kv_raw"], d["sink"], p["m_prime"], p["n_win"],
                          d["scale"])
    torch.cuda.synchronize()
    C, Z, B = to64(d["C"]), to64(d["Z"]), to64(d["B"])
    wCc = O.compress_pool(C, Z, B, p["m_prime"])
    assert_close(Cc[0], wCc, torch.bfloat16, "Ccomp")
    rows = np.unique(np.concatenate([np.arange(0, 4), [126, 127, 128, 129, 255, 256],
                                     np.arange(131068, 131072),
                                     np.random.default_rng(2).integers(0, p["n"], 16)]))
    q_rows = d["q"][torch.tensor(rows, device=DEV)]
    Cc16 = torch.tensor(wCc, dtype=torch.float32).to(torch.bfloat16)
    want = O.hca_attend(to64(q_rows), to64(Cc16), C, 0, to64(d["sink"]), rows, p["m_prime"], p["n_win"],
                        d["scale"])
    assert_close(out[0, torch.tensor(rows, device=DEV)], want, torch.bfloat16, "out")


def test_hca_decode_one_million_context_sampled():
    # HCA attention at the 1M-token decode shape: 8 sequences, 8192 completed
    # entries (m' = 128) plus the 128-row window, one query each (the split
    # launch and its combine), checked on two sequences
    say("hca decode 8 x 8192 entries (sampled sequences)")
    b, ne, c, nh, mp, nw = 8, 8192, 512, 64, 128, 128
    gen = torch.Generator(device=DEV).manual_seed(53)
    Cc = (torch.randn((b, ne, c), generator=gen, device=DEV) / math.sqrt(c)).to(torch.bfloat16)
    win = (torch.randn((b, nw, c), generator=gen, device=DEV) / math.sqrt(c)).to(torch.bfloat16)
    q = (torch.randn((b, 1, nh, c), generator=gen, device=DEV) / math.sqrt(c)).to(torch.bfloat16)
    sink = torch.randn((nh,), generator=gen, device=DEV)
    t = ne * mp + 5          # (t + 1) // m' = 8192 entries visible
    out = L.hca_attend(q, Cc, win, sink, t, mp, nw, raw_pos0=t - nw + 1)
    torch.cuda.synchronize()
    for s in (0, b - 1):
        want = O.hca_attend(to64(q[s].cpu()), to64(Cc[s].cpu()), to64(win[s].cpu()), t - nw + 1, to64(sink.cpu()),
                            [t], mp, nw, 1 / math.sqrt(c))
        assert_close(out[s], want, torch.bfloat16, f"seq {s}")


# ------------------------------------------------------------- whole layer --

def test_csa_layer_tiny_fp32_end_to_end():
    # compressor -> indexer (given keys) -> attention, all on the GPU
    say("csa layer tiny fp32 end to end")
    d = synth.tiny_inputs()
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    Cc = L.csa_compress(*(g(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    idx = L.csa_index_topk(g(d["qI"]), g(d["w"]), g(d["KIcomp"]), 0, m, k)
    out = L.csa_attend(g(d["q"]), Cc, idx, g(d["kv_raw"]), g(d["sink"]), 0, m, nw, d["scale"])
    torch.cuda.synchronize()
    wCc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    widx, osc, vis = _oracle_index(d["qI"], d["w"], d["KIcomp"], np.arange(n), m, k)
    assert assert_index_sets(idx[0].cpu().numpy(), widx, osc, vis, k) == 0
    want = O.csa_attend(to64(d["q"]), wCc, widx, to64(d["kv_raw"]), 0, to64(d["sink"]), np.arange(n), nw,
                        d["scale"], m)
    assert_close(out[0], want, torch.float32)


def test_future_tokens_do_not_change_gpu_outputs():
    say("causality on the GPU at t = 3, 4, 7, 8")
    d = synth.tiny_inputs(n=16)
    p = d["params"]
    m, k, nw = p["m"], p["k"], 4

    def run(dd):
        Cc = L.csa_compress(*(g(dd[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
        KI = L.csa_compress(*(g(dd[x]) for x in ("ICa", "ICb", "IZa", "IZb", "Ba16", "Bb16")), m)
        idx = L.csa_index_topk(g(dd["qI"]), g(dd["w"]), KI, 0, m, k)
        return L.csa_attend(g(dd["q"]), Cc, idx, g(dd["Ca"]), g(d["sink"]), 0, m, nw, d["scale"]).cpu()

    gen = torch.Generator().manual_seed(61)
    base = dict(d)
    for x in ("ICa", "ICb", "IZa", "IZb"):
        base[x] = torch.randn((16, 16), generator=gen)
    base["Ba16"] = torch.randn((m, 16), generator=gen) * 0.1
    base["Bb16"] = torch.randn((m, 16), generator=gen) * 0.1
    ref = run(base)
    for t in (3, 4, 7, 8):
        mix = dict(base)
        for x in ("Ca", "Cb", "Za", "Zb", "q", "qI", "w", "ICa", "ICb", "IZa", "IZb"):
            a = base[x].clone()
            a[t + 1:] = torch.randn(a[t + 1:].shape, generator=gen)
            mix[x] = a
        got = run(mix)
        assert torch.equal(got[0, t], ref[0, t]), t


def test_results_are_bitwise_reproducible():
    say("determinism")
    d = synth.prefill_inputs(n=512, seed=71)
    p = d["params"]
    args = [g(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")]
    outs = []
    for _ in range(2):
        Cc = L.csa_compress(*args, 4)
        idx = L.csa_index_topk(g(d["qI"]), g(d["w"]), g(d["KIcomp"][:128]), 0, 4, 64)
        o = L.csa_attend(g(d["q"]), Cc, idx, g(d["kv_raw"]), g(d["sink"]), 0, 4, p["n_win"])
        outs.append((Cc.cpu(), idx.cpu(), o.cpu()))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


# ----------------------------------------------------------------- decode --

class GpuDecode:
    """Decode driver over the library: caller-side state appends (row copies),
    the compressor when a block completes, then indexer/top-k and attention."""

    def __init__(self, Cc, KI, n_comp, window, win_pos0, prev, biases, m, n_win, k, sink, scale):
        self.Cc, self.KI, self.n_comp = Cc, KI, n_comp
        self.win, self.win_pos0 = window, win_pos0
        self.prev = dict(prev)
        self.B = biases
        self.m, self.n_win, self.k, self.sink, self.scale = m, n_win, k, sink, scale
        b = Cc.shape[0]
        self.tail = {key: torch.empty((b, m, (Cc if key[0] != "I" else KI).shape[2]), dtype=Cc.dtype,
                                      device=DEV) for key in ("Ca", "Cb", "Za", "Zb", "ICa", "ICb", "IZa", "IZb")}

    def step(self, t, tok, q, qI, w):
        m = self.m
        for key in self.tail:
            self.tail[key][:, t % m].copy_(tok[key])
        self.win[:, t - self.win_pos0].copy_(tok["Ca"])
        if (t + 1) % m == 0:
            e = (t + 1) // m - 1
            L.csa_compress(self.tail["Ca"], self.tail["Cb"], self.tail["Za"], self.tail["Zb"], self.B["Ba"],
                           self.B["Bb"], m, prev_Cb=self.prev["Cb"], prev_Zb=self.prev["Zb"],
                           out=self.Cc[:, e:e + 1])
            L.csa_compress(self.tail["ICa"], self.tail["ICb"], self.tail["IZa"], self.tail["IZb"], self.B["IBa"],
                           self.B["IBb"], m, prev_Cb=self.prev["ICb"], prev_Zb=self.prev["IZb"],
                           out=self.KI[:, e:e + 1])
            for key in ("Cb", "Zb", "ICb", "IZb"):
                self.prev[key] = self.tail[key].clone()
            self.n_comp = e + 1
        idx = L.csa_index_topk(qI, w, self.KI, t, m, self.k, n_comp=self.n_comp)
        out = L.csa_attend(q, self.Cc, idx, self.win, self.sink, t, m, self.n_win, self.scale,
                           raw_pos0=self.win_pos0, n_comp=self.n_comp)
        return idx, out


def test_decode_steps_match_oracle_decode_state():
    say("decode continuity vs oracle state (b=2, 64 heads, c=512)")
    b, m, k, nw, n0, steps, c, cI, nh, nI = 2, 4, 24, 32, 150, 11, 512, 128, 64, 64
    n = n0 + steps
    gen = torch.Generator().manual_seed(81)
    rnd = lambda *s: (torch.randn(s, generator=gen) / math.sqrt(s[-1])).to(torch.bfloat16)
    st = {key: rnd(b, n, c) for key in ("Ca", "Cb", "Za", "Zb")}
    st.update({key: rnd(b, n, cI) for key in ("ICa", "ICb", "IZa", "IZb")})
    B = {"Ba": rnd(m, c), "Bb": rnd(m, c), "IBa": rnd(m, cI), "IBb": rnd(m, cI)}
    q, qI = rnd(b, n, nh, c), rnd(b, n, nI, cI)
    w = torch.nn.functional.softplus(torch.randn((b, n, nI), generator=gen))
    sink = torch.randn(nh, generator=gen)
    scale = 1 / math.sqrt(c)
    # prefill of the first n0 tokens on the GPU, caches with room to grow
    cap = n // m + 4
    Cc = torch.zeros((b, cap, c), dtype=torch.bfloat16, device=DEV)
    KI = torch.zeros((b, cap, cI), dtype=torch.bfloat16, device=DEV)
    ne0 = n0 // m
    Cc[:, :ne0] = L.csa_compress(*(g(st[x][:, :n0]) for x in ("Ca", "Cb", "Za", "Zb")), g(B["Ba"]), g(B["Bb"]), m)
    KI[:, :ne0] = L.csa_compress(*(g(st[x][:, :n0]) for x in ("ICa", "ICb", "IZa", "IZb")), g(B["IBa"]),
                                 g(B["IBb"]), m)
    blk = slice(m * (ne0 - 1), m * ne0)
    prev = {x: g(st[x][:, blk]) for x in ("Cb", "Zb", "ICb", "IZb")}
    win_pos0 = max(0, n0 - nw)
    window = torch.zeros((b, n - win_pos0, c), dtype=torch.bfloat16, device=DEV)
    window[:, : n0 - win_pos0] = g(st["Ca"][:, win_pos0:n0])
    drv = GpuDecode(Cc, KI, ne0, window, win_pos0, prev, {x: g(v) for x, v in B.items()}, m, nw, k, g(sink), scale)
    # the tail of an incomplete block must already hold its rows
    for t in range(m * ne0, n0):
        for key in drv.tail:
            drv.tail[key][:, t % m].copy_(g(st[key][:, t]))
    states = []
    for s in range(b):
        o = O.CsaDecodeState(m=m, n_win=nw, c=c, c_I=cI)
        for t in range(n0):
            o.append({x: to64(st[x][s, t]) for x in st}, {x: to64(v) for x, v in B.items()})
        states.append(o)
    chained = tie_steps = 0
    for t in range(n0, n):
        idx, out = drv.step(t, {x: g(st[x][:, t]) for x in st}, g(q[:, t:t + 1]), g(qI[:, t:t + 1]),
                            g(w[:, t:t + 1]))
        torch.cuda.synchronize()
        for s in range(b):
            states[s].append({x: to64(st[x][s, t]) for x in st}, {x: to64(v) for x, v in B.items()})
            oi, oo = states[s].query(to64(q[s, t]), to64(qI[s, t]), to64(w[s, t]), to64(sink), k, scale)
            KIo = np.array(states[s].KIcomp)
            osc = O.index_scores(to64(qI[s, t])[None], to64(w[s, t])[None], KIo, [t], m)
            vis = [min((t + 1) // m, KIo.shape[0])]
            assert_index_sets(idx[s].cpu().numpy(), oi[None], osc, vis, k, f"t={t} seq {s}")
            # attention against the oracle state's own entries with the oracle's selection
            Cco = np.array(states[s].Ccomp)
            Cco16 = torch.tensor(Cco, dtype=torch.float32).to(torch.bfloat16)
            pos0 = states[s].window[0][0]
            raw = np.stack([r for _, r in states[s].window])
            want = O.csa_attend(to64(q[s, t])[None], to64(Cco16), oi[None], raw, pos0, to64(sink), [t], nw,
                                scale, m)
            # always: the GPU attention step on the oracle's selection (the
            # chained output uses the GPU's own selection, which may settle a
            # near-tie the other way)
            o_sel = L.csa_attend(g(q[s:s + 1, t:t + 1]), drv.Cc[s:s + 1], g(torch.tensor(oi[None, None], dtype=torch.int32)),
                                 drv.win[s:s + 1], drv.sink, t, m, nw, scale, raw_pos0=drv.win_pos0,
                                 n_comp=drv.n_comp)
            torch.cuda.synchronize()
            assert_close(o_sel[0], want, torch.bfloat16, f"t={t} seq {s}, oracle selection")
            if set(idx[s, 0].cpu().numpy().tolist()) == set(oi.tolist()):
                assert_close(out[s], want, torch.bfloat16, f"t={t} seq {s}, chained")
                chained += 1
            else:
                tie_steps += 1
    print(f"[ties] decode continuity: {tie_steps} of {chained + tie_steps} (step, sequence) selections settled a "
          f"near-tie differently; the chained output was compared on the other {chained}", flush=True)
    assert chained >= (chained + tie_steps) // 2
    # the caches match the oracle's entries
    for s in range(b):
        assert_close(drv.Cc[s, : drv.n_comp], np.array(states[s].Ccomp), torch.bfloat16, "Ccomp")
        assert_close(drv.KI[s, : drv.n_comp], np.array(states[s].KIcomp), torch.bfloat16, "KIcomp")


def test_decode_one_million_context_sampled():
    say("decode 8 x 1M history (sampled sequences)")
    d = synth.decode_inputs(device=DEV)
    p = d["params"]
    b, hist, m, nh, c, nw, nI, cI, k, steps = (p["b"], p["history"], p["m"], p["n_h"], p["c"], p["n_win"],
                                               p["n_hI"], p["c_I"], p["k"], p["steps"])
    ne0 = d["n_comp0"]
    prev = {"Cb": d["prev_Cb"], "Zb": d["prev_Zb"], "ICb": d["prev_ICb"], "IZb": d["prev_IZb"]}
    B = {x: d[x] for x in ("Ba", "Bb", "IBa", "IBb")}
    drv = GpuDecode(d["Ccomp"], d["KIcomp"], ne0, d["window"], d["window_pos0"], prev, B, m, nw, k, d["sink"],
                    d["scale"])
    results = []
    for i in range(steps):
        t = hist + i
        idx, out = drv.step(t, {x: d["tok"][x][i] for x in d["tok"]}, d["q"][i], d["qI"][i], d["w"][i])
        results.append((t, idx.clone(), out.clone()))
    torch.cuda.synchronize()
    for s in (0, b - 1):
        KI = to64(d["KIcomp"][s, :ne0])
        # the entry completed by the last step, computed by the oracle from the tokens
        toks = {x: to64(d["tok"][x][:, s]) for x in d["tok"]}
        e_new = O.compress_overlap(toks["Ca"], toks["Cb"], toks["Za"], toks["Zb"], to64(d["Ba"]), to64(d["Bb"]),
                                   m, to64(d["prev_Cb"][s]), to64(d["prev_Zb"][s]))
        ki_new = O.compress_overlap(toks["ICa"], toks["ICb"], toks["IZa"], toks["IZb"], to64(d["IBa"]),
                                    to64(d["IBb"]), m, to64(d["prev_ICb"][s]), to64(d["prev_IZb"][s]))
        assert_close(d["Ccomp"][s, ne0:ne0 + 1], e_new, torch.bfloat16, "new entry")
        assert_close(d["KIcomp"][s, ne0:ne0 + 1], ki_new, torch.bfloat16, "new key")
        for i in (0, steps - 1):
            t, idx, out = results[i]
            n_comp = (t + 1) // m
            KIt = np.concatenate([KI, ki_new])[:n_comp]
            qI = to64(d["qI"][i][s, 0])[None]
            w = to64(d["w"][i][s, 0])[None]
            sc = O.index_scores(qI, w, KIt, [t], m)
            oi = O.topk_select(sc[0], n_comp, k)
            assert_index_sets(idx[s].cpu().numpy(), oi[None], sc, [n_comp], k, f"t={t} seq {s}")
            # attention with the oracle's selection: gather those rows only
            rows = torch.tensor(oi[oi >= 0], device=DEV)
            Csel = to64(d["Ccomp"][s, rows[rows < ne0]])
            if (oi >= ne0).any():
                Csel = np.concatenate([Csel, to64(torch.tensor(e_new, dtype=torch.float32).to(torch.bfloat16))])
            win_rows = to64(d["window"][s])
            want = O.csa_attend(to64(d["q"][i][s]), Csel, np.arange(len(Csel))[None], win_rows, d["window_pos0"],
                                to64(d["sink"]), [t], nw, d["scale"])
            # always: the GPU attention step over the whole cache with the
            # oracle's selection; the chained output too when the GPU chose
            # the same set (a near-tie may be settled the other way)
            o_sel = L.csa_attend(d["q"][i][s:s + 1], d["Ccomp"][s:s + 1], g(torch.tensor(oi[None, None], dtype=torch.int32)),
                                 d["window"][s:s + 1], d["sink"], t, m, nw, d["scale"], raw_pos0=d["window_pos0"],
                                 n_comp=n_comp)
            torch.cuda.synchronize()
            assert_close(o_sel[0], want, torch.bfloat16, f"t={t} seq {s}, oracle selection")
            if set(idx[s, 0].cpu().numpy().tolist()) == set(oi.tolist()):
                assert_close(out[s], want, torch.bfloat16, f"t={t} seq {s}, chained")
            else:
                print(f"[ties] t={t} seq {s}: the GPU settled a near-tie differently; chained output not compared",
                      flush=True)


def test_graph_replay_matches_eager():
    # The library allocates nothing and records no memset, so whole layer
    # steps can be captured in a HIP graph: a prefill-shaped step (both
    # compressors, scoring with fused selection, attention, query norm and
    # rotation, the output's in-place back-rotation, the grouped output
    # projection) and a
    # decode-shaped step (streaming scorer, threshold top-k, split attention)
    # are replayed three times, with eager work between the replays, and every
    # replay must reproduce the eager results bit for bit.
    say("graph capture and replay")
    m, nw = 4, 128
    p = synth.prefill_inputs(n=1024, device=DEV, k=64)
    n, c, k = p["params"]["n"], p["params"]["c"], p["params"]["k"]
    ne = n // m
    Cc = torch.empty((1, ne, c), dtype=torch.bfloat16, device=DEV)
    KI = torch.empty((1, ne, 128), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((1, n, k), dtype=torch.int32, device=DEV)
    out = torch.empty((1, n, 64, c), dtype=torch.bfloat16, device=DEV)
    lib = L.load_library()
    wsI = torch.empty(max(lib.csa_index_topk_workspace_size(1, n, ne, k), 256), dtype=torch.uint8, device=DEV)
    wsA = torch.empty(max(lib.csa_attend_workspace_size(1, n, 0, ne, 64, c, k, m, nw, 1), 256),
                      dtype=torch.uint8, device=DEV)
    # decode-shaped: 2 sequences, 20000 entries, one query each
    gen = torch.Generator().manual_seed(31)
    b, nd, kd = 2, 20000, 512
    td = nd * m - 1
    dq = g(torch.randn((b, 1, 64, c), generator=gen) / math.sqrt(c)).to(torch.bfloat16)
    dqI = g(torch.randn((b, 1, 64, 128), generator=gen) / math.sqrt(128)).to(torch.bfloat16)
    dw = g(torch.nn.functional.softplus(torch.randn((b, 1, 64), generator=gen)))
    dKI = g(torch.randn((b, nd, 128), generator=gen) / math.sqrt(128)).to(torch.bfloat16)
    dCc = g(torch.randn((b, nd, c), generator=gen) / math.sqrt(c)).to(torch.bfloat16)
    dwin = g(torch.randn((b, nw, c), generator=gen) / math.sqrt(c)).to(torch.bfloat16)
    dsink = g(torch.randn(64, generator=gen))
    didx = torch.empty((b, 1, kd), dtype=torch.int32, device=DEV)
    dout = torch.empty((b, 1, 64, c), dtype=torch.bfloat16, device=DEV)
    dwsI = torch.empty(max(lib.csa_index_topk_workspace_size(b, 1, nd, kd), 256), dtype=torch.uint8, device=DEV)
    dwsA = torch.empty(max(lib.csa_attend_workspace_size(b, 1, td, nd, 64, c, kd, m, nw, 1), 256),
                       dtype=torch.uint8, device=DEV)
    _, gq = synth.norm_rope_inputs(1, 1, c, seed=71, device=DEV)
    _, WG, WO = synth.out_proj_inputs(1, 64, c, 8, 256, 512, seed=72, device=DEV)
    qn = torch.empty_like(p["q"])
    mid = torch.empty((n, 8 * 256), dtype=torch.bfloat16, device=DEV)
    proj = torch.empty((n, 512), dtype=torch.bfloat16, device=DEV)
    outs = (Cc, KI, idx, out, didx, dout, qn, mid, proj)

    def body(s):
        L.csa_compress(*(p[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m, out=Cc, stream=s)
        L.csa_compress(*(p[x] for x in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")), m, out=KI, stream=s)
        L.csa_index_topk(p["qI"], p["w"], KI, 0, m, k, idx=idx, workspace=wsI, stream=s)
        L.csa_attend(p["q"], Cc, idx, p["kv_raw"], p["sink"], 0, m, nw, out=out, workspace=wsA, stream=s)
        L.csa_norm_rope(p["q"], gq, 1e-6, 64, 10000.0, 0, 1, out=qn, stream=s)
        L.csa_norm_rope(out[0], None, 0.0, 64, 10000.0, 0, -1, out=out[0], stream=s)
        L.csa_grouped_out_proj(out[0], WG, WO, mid=mid, out=proj, stream=s)
        L.csa_index_topk(dqI, dw, dKI, td, m, kd, idx=didx, workspace=dwsI, stream=s)
        L.csa_attend(dq, dCc, didx, dwin, dsink, td, m, nw, raw_pos0=td - nw + 1, out=dout, workspace=dwsA,
                     stream=s)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        body(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        body(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"replay {rep}: output {i} differs from the eager run"
    # and the eager results are right: the decode selection against the oracle
    for sq in range(b):
        sc = O.index_scores(to64(dqI[sq, 0])[None], to64(dw[sq, 0])[None], to64(dKI[sq]), [td], m)
        oi = O.topk_select(sc[0], nd, kd)
        assert_index_sets(didx[sq].cpu().numpy(), oi[None], sc, [nd], kd, f"graph decode seq {sq}")


# ------------------------------------------------ RMSNorm and partial RoPE --

@pytest.mark.parametrize("dtype,rows,heads,c,rd,gain,pos0,step", [
    (torch.float32, 37, 3, 64, 16, True, 0, 1),              # heads per wave, ragged last pass
    (torch.bfloat16, 6, 64, 512, 64, True, 1000, 1),         # query heads of a prefill block
    (torch.bfloat16, 300, 1, 512, 64, True, 0, 4),           # compressed entries at m * s
    (torch.bfloat16, 5, 64, 512, 64, False, -1048579, -1),   # output turned back by -t near 2^20
    (torch.bfloat16, 8, 64, 512, 64, True, 1048576, 0),      # one decode step of 8 sequences
    (torch.bfloat16, 9, 2, 1024, 128, True, 3, 7),           # two chunks per lane
    (torch.bfloat16, 4, 1, 2048, 512, True, -5, 3),          # four chunks per lane, widest rotation
    (torch.float32, 7, 5, 1024, 0, True, 0, 1),              # norm only
    (torch.float32, 3, 1, 520, 64, False, 9, 1),             # rotation only, ragged chunk count
])
def test_norm_rope(dtype, rows, heads, c, rd, gain, pos0, step):
    say(f"norm_rope {dtype} rows={rows} heads={heads} c={c} rope={rd} gain={gain} pos0={pos0} step={step}")
    x, gamma = synth.norm_rope_inputs(rows, heads, c, dtype, seed=rows * 7 + c, gain=gain)
    out = L.csa_norm_rope(g(x), None if gamma is None else g(gamma), 1e-6, rd, 10000.0, pos0, step)
    torch.cuda.synchronize()
    pos = pos0 + step * np.arange(rows)
    want = O.norm_rope(to64(x), None if gamma is None else to64(gamma), 1e-6, pos, rd, 10000.0)
    assert_close(out, want, dtype, "norm_rope")


@pytest.mark.parametrize("dtype,c,rd", [
    (torch.bfloat16, 512, 64),     # the attention output's back-rotation
    (torch.float32, 520, 62),      # rotated part starting inside a 16-byte chunk
    (torch.bfloat16, 64, 0),       # nothing rotated: unchanged
])
def test_norm_rope_rotation_only_in_place(dtype, c, rd):
    # no gain and out == x: only the chunks holding rotated dimensions are
    # read and written; every other value must stay bit for bit
    say(f"norm_rope rotation only, in place {dtype} c={c} rope={rd}")
    rows, heads = 11, 5
    x, _ = synth.norm_rope_inputs(rows, heads, c, dtype, seed=c + rd, gain=False)
    xd = g(x)
    got = L.csa_norm_rope(xd, None, 0.0, rd, 10000.0, -40, -3, out=xd)
    torch.cuda.synchronize()
    assert got.data_ptr() == xd.data_ptr()
    got = got.cpu()
    assert torch.equal(got[..., :c - rd], x[..., :c - rd])
    want = O.rope(to64(x), -40 - 3 * np.arange(rows), rd, 10000.0)
    assert_close(got, want, dtype, "rotation in place")


def test_norm_rope_in_place_on_strided_rows():
    # the first vector of every cache row, updated in place through the row
    # stride; the second vector of each row must not move
    say("norm_rope in place, strided rows")
    rows, c = 33, 512
    x, gamma = synth.norm_rope_inputs(rows, 2, c, torch.bfloat16, seed=77)
    xd = g(x)
    lib = L.load_library()
    rc = lib.csa_norm_rope(xd.data_ptr(), 2 * c, xd.data_ptr(), 2 * c, g(gamma).data_ptr(), 1e-6, rows, 1, c,
                           64, 10000.0, 12, 4, L.CSA_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = xd.cpu()
    assert torch.equal(got[:, 1], x[:, 1])
    want = O.norm_rope(to64(x[:, 0]), to64(gamma), 1e-6, 12 + 4 * np.arange(rows), 64, 10000.0)
    assert_close(got[:, 0], want, torch.bfloat16, "in place")


def _norm_rope_layer_case(n, nh, k, seed):
    d = synth.prefill_inputs(n=n, seed=seed, n_h=nh, k=k, unscaled=True)
    _, gq = synth.norm_rope_inputs(1, 1, 512, seed=seed + 1)
    _, gk = synth.norm_rope_inputs(1, 1, 512, seed=seed + 2)
    m = 4
    Cc = torch.tensor(O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m),
                      dtype=torch.float32)
    idx = torch.tensor(_oracle_idx_for(d["KIcomp"], d["qI"], d["w"], np.arange(n), m, k), dtype=torch.int32)
    return d, gq, gk, Cc, idx, m


def _norm_rope_layer_gpu(q, Cc, idx, raw, sink, gq, gk, m, nw, scale, eps, rd, base):
    qn = L.csa_norm_rope(g(q), g(gq), eps, rd, base, 0, 1)
    Cn = L.csa_norm_rope(g(Cc), g(gk), eps, rd, base, 0, m)
    Rn = L.csa_norm_rope(g(raw), g(gk), eps, rd, base, 0, 1)
    o = L.csa_attend(qn[None], Cn[None], g(idx)[None], Rn[None], g(sink), 0, m, nw, scale)[0]
    L.csa_norm_rope(o, None, 0.0, rd, base, 0, -1, out=o)
    torch.cuda.synchronize()
    return o


def test_csa_layer_with_norm_and_rope_fp32():
    # the composition (positions of queries, entries at m*s and window rows,
    # the output turned back by -t) against the oracle's composed definition,
    # float32 throughout so that the strict float32 bound applies
    n, nh, k, nw = 128, 64, 16, 48
    say(f"csa layer with norm and rope, float32 n={n} n_h={nh} k={k} n_win={nw}")
    d, gq, gk, Cc, idx, m = _norm_rope_layer_case(n, nh, k, 43)
    f = lambda t: t.to(torch.float32)
    eps, rd, base = 1e-6, 64, 10000.0
    o = _norm_rope_layer_gpu(f(d["q"]), Cc, idx, f(d["kv_raw"]), d["sink"], gq, gk, m, nw, d["scale"], eps, rd,
                             base)
    want = O.csa_attend_rope(to64(d["q"]), to64(Cc), idx.numpy(), to64(d["kv_raw"]), 0, to64(d["sink"]),
                             np.arange(n), nw, d["scale"], m, to64(gq), to64(gk), eps, rd, base)
    assert_close(o, want, torch.float32, "layer with norm and rope, float32")


def test_csa_layer_with_norm_and_rope_bf16():
    # the bf16 production path: normalised queries, entries and window rows
    # and the output are stored in bf16 between the calls.  The reference
    # composes the oracle's pieces with the same round-to-nearest-even
    # storage at those points (torch conversion), so the bound measures the
    # kernels, not the storage format (four bf16 stores alone move single
    # outputs by up to 3% of their row RMS at this shape)
    n, nh, k, nw = 512, 64, 64, 128
    say(f"csa layer with norm and rope, bf16 n={n} n_h={nh} k={k}")
    d, gq, gk, Cc, idx, m = _norm_rope_layer_case(n, nh, k, 43)
    Cc = Cc.to(torch.bfloat16)
    eps, rd, base = 1e-6, 64, 10000.0
    o = _norm_rope_layer_gpu(d["q"], Cc, idx, d["kv_raw"], d["sink"], gq, gk, m, nw, d["scale"], eps, rd, base)
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    t = np.arange(n)
    qn = st(O.norm_rope(to64(d["q"]), to64(gq), eps, t, rd, base))
    Cn = st(O.norm_rope(to64(Cc), to64(gk), eps, m * np.arange(Cc.shape[0]), rd, base))
    Rn = st(O.norm_rope(to64(d["kv_raw"]), to64(gk), eps, t, rd, base))
    att = st(O.csa_attend(qn, Cn, idx.numpy(), Rn, 0, to64(d["sink"]), t, nw, d["scale"], m))
    want = O.rope(att, -t, rd, base)
    lo = want.shape[-1] - rd
    assert_close(o[..., :lo], want[..., :lo], torch.bfloat16, "layer with norm and rope, bf16, unrotated dims")
    # rotated dims: the output was stored in bf16 before its rotation, so each
    # element also carries the storage error of its pair partner; a rotation
    # keeps the pair's norm, so the two carried errors (at most one bf16 step
    # each, 2^-7 of the element) add at most 2^-7 of the pair's norm
    got = to64(o)
    rms = np.sqrt(np.mean(want ** 2, axis=-1, keepdims=True))
    pair = np.sqrt(want[..., lo::2] ** 2 + want[..., lo + 1::2] ** 2).repeat(2, axis=-1)
    bound = np.maximum(2e-2 * rms, bf16_ulp(want[..., lo:]) + 2.0 ** -7 * pair)
    ratio = np.abs(got[..., lo:] - want[..., lo:]) / bound
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    print(f"[margin] rotated dims: worst err/bound {ratio[i]:.3f}", flush=True)
    assert ratio[i] <= 1.0, ("rotated dims", i, got[..., lo:][i], want[..., lo:][i], bound[i])


def test_attend_norm_rope_fused_prefill():
    # the query norm and rotation done inside the attention's Q load and the
    # -t rotation of the output in its epilogue: queries rounded to bf16 after
    # norm and rotation (the kernel's operand precision), the output stored
    # once, after the back-rotation
    n, nh, k, nw = 512, 64, 64, 128
    say(f"attend with fused query norm and rope, prefill n={n} n_h={nh} k={k}")
    d, gq, gk, Cc, idx, m = _norm_rope_layer_case(n, nh, k, 47)
    Cc = Cc.to(torch.bfloat16)
    eps, rd, base = 1e-6, 64, 10000.0
    Cn = L.csa_norm_rope(g(Cc), g(gk), eps, rd, base, 0, m)
    Rn = L.csa_norm_rope(g(d["kv_raw"]), g(gk), eps, rd, base, 0, 1)
    o = L.csa_attend_norm_rope(g(d["q"])[None], g(gq), eps, rd, base, Cn[None], g(idx)[None], Rn[None],
                               g(d["sink"]), 0, m, nw, d["scale"])[0]
    torch.cuda.synchronize()
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    t = np.arange(n)
    qn = st(O.norm_rope(to64(d["q"]), to64(gq), eps, t, rd, base))
    Cw = st(O.norm_rope(to64(Cc), to64(gk), eps, m * np.arange(Cc.shape[0]), rd, base))
    Rw = st(O.norm_rope(to64(d["kv_raw"]), to64(gk), eps, t, rd, base))
    att = O.csa_attend(qn, Cw, idx.numpy(), Rw, 0, to64(d["sink"]), t, nw, d["scale"], m)
    assert_close(o, O.rope(att, -t, rd, base), torch.bfloat16, "fused norm and rope, prefill")


def test_attend_norm_rope_fused_prefill_full_size_sampled():
    # the launch the benchmark's fused step times (n = 8192, 64 heads,
    # k = 512, window 128) on oracle indices and oracle-normalised entries
    # and window rows; sampled queries against the oracle
    say("attend with fused query norm and rope, prefill n=8192 (oracle indices, sampled queries)")
    d = synth.prefill_inputs()
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    _, gq = synth.norm_rope_inputs(1, 1, 512, seed=46)
    _, gk = synth.norm_rope_inputs(1, 1, 512, seed=47)
    eps, rd, base = 1e-6, 64, 10000.0
    st = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)
    Cc = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    Cn = st(O.norm_rope(Cc, to64(gk), eps, m * np.arange(Cc.shape[0]), rd, base))
    Rn = st(O.norm_rope(to64(d["kv_raw"]), to64(gk), eps, np.arange(n), rd, base))
    idx = _oracle_idx_for(d["KIcomp"], d["qI"], d["w"], np.arange(n), m, k)
    out = L.csa_attend_norm_rope(g(d["q"])[None], g(gq), eps, rd, base, g(Cn)[None],
                                 g(torch.tensor(idx, dtype=torch.int32))[None], g(Rn)[None], g(d["sink"]), 0, m, nw,
                                 d["scale"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 6), [127, 128, 2047, 2048, 2051], np.arange(8188, 8192),
                                     np.random.default_rng(2).integers(0, n, 24)]))
    qn = to64(st(O.norm_rope(to64(d["q"][rows]), to64(gq), eps, rows, rd, base)))
    att = O.csa_attend(qn, to64(Cn), idx[rows], to64(Rn), 0, to64(d["sink"]), rows, nw, d["scale"], m)
    assert_close(out[0, rows], O.rope(att, -rows, rd, base), torch.bfloat16, "fused norm and rope, n=8192")


def test_attend_norm_rope_fused_chunk_batch_two_groups():
    # a later chunk of two sequences (queries at t0 .. t0 + n_q - 1, window
    # rows from t0 - n_win + 1), two 64-head groups, padded index lists
    b, n_q, t0, nh, k, nw, m = 2, 96, 300, 128, 32, 64, 4
    say(f"attend with fused query norm and rope, chunk b={b} n_q={n_q} t0={t0} n_h={nh} k={k}")
    gen = torch.Generator().manual_seed(61)
    n_comp = (t0 + n_q) // m
    raw_pos0 = t0 - nw + 1
    n_raw = t0 + n_q - raw_pos0
    q = (2.5 * torch.randn((b, n_q, nh, 512), generator=gen)).to(torch.bfloat16)
    gq = 0.5 + torch.rand(512, generator=gen)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, n_raw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(nh, generator=gen)
    t_pos = t0 + np.arange(n_q)
    idx = np.full((b, n_q, k), -1, dtype=np.int32)
    for s_ in range(b):
        for r in range(n_q):
            vis = (t_pos[r] + 1) // m
            take = min(k - (r % 5), vis)     # some lists padded with -1
            idx[s_, r, :take] = np.sort(torch.randperm(vis, generator=gen)[:take].numpy())
    eps, rd, base = 1e-6, 64, 10000.0
    out = L.csa_attend_norm_rope(g(q), g(gq), eps, rd, base, g(Cc), g(torch.tensor(idx)), g(raw), g(sink), t0, m,
                                 nw, 1 / math.sqrt(512), raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    for s_ in range(b):
        qn = st(O.norm_rope(to64(q[s_]), to64(gq), eps, t_pos, rd, base))
        att = O.csa_attend(qn, to64(Cc[s_]), idx[s_], to64(raw[s_]), raw_pos0, to64(sink), t_pos, nw,
                           1 / math.sqrt(512), m)
        assert_close(out[s_], O.rope(att, -t_pos, rd, base), torch.bfloat16, f"seq {s_}")


@pytest.mark.parametrize("nh,rd,t", [
    (64, 64, 2002),          # the model's rotary width
    (128, 0, 4099),          # norm only, two head groups
    (64, 256, (1 << 20) + 3),  # wide rotation at a large position
    (64, 510, 777),          # every dimension but the first pair rotated
])
def test_attend_norm_rope_fused_decode_split(nh, rd, t):
    # one query per sequence: the entries are split over workgroups, each
    # partial output turned back by -t before the merge
    say(f"attend with fused query norm and rope, decode n_h={nh} rope_dims={rd} t={t}")
    m, k, nw, b = 4, 96, 128, 2
    n_comp = min((t + 1) // m, 600)    # the cache holds the last completed entries only
    gen = torch.Generator().manual_seed(53 + rd)
    q = (3.0 * torch.randn((b, 1, nh, 512), generator=gen)).to(torch.bfloat16)
    gq = 0.5 + torch.rand(512, generator=gen)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(nh, generator=gen)
    idx = torch.stack([torch.sort(torch.randperm(n_comp, generator=gen)[:k]).values for _ in range(b)])
    idx = idx.to(torch.int32)[:, None, :]
    raw_pos0 = t - nw + 1
    eps, base = 1e-6, 10000.0
    out = L.csa_attend_norm_rope(g(q), g(gq), eps, rd, base, g(Cc), g(idx), g(raw), g(sink), t, m, nw,
                                 1 / math.sqrt(512), raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    for s in range(b):
        qn = st(O.norm_rope(to64(q[s]), to64(gq), eps, [t], rd, base))
        att = O.csa_attend(qn, to64(Cc[s]), idx[s].numpy(), to64(raw[s]), raw_pos0, to64(sink), [t], nw,
                           1 / math.sqrt(512), m)
        assert_close(out[s], O.rope(att, -np.array([t]), rd, base), torch.bfloat16, f"seq {s}")


# ------------------------------------------------ grouped output projection --

def _check_out_proj(o, WG, WO, what):
    g = WG.shape[0]
    mid, out = L.csa_grouped_out_proj(g_(o), g_(WG), g_(WO))
    torch.cuda.synchronize()
    want_mid, _ = O.grouped_out_proj(to64(o), to64(WG), to64(WO), g)
    assert_close(mid, want_mid, torch.bfloat16, f"{what}: intermediate")
    # the intermediate is stored in bf16 between the two products: the
    # reference rounds the oracle's at the same point
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    _, want = O.grouped_out_proj(to64(o), to64(WG), to64(WO), g, mid_round=st)
    assert_close(out, want, torch.bfloat16, f"{what}: output")


g_ = g


@pytest.mark.parametrize("n,n_h,c,g,d_g,d", [
    (37, 8, 64, 2, 192, 320),      # ragged rows and columns, 4 and 6 K stages
    (5, 2, 32, 1, 128, 64),        # one and two K stages
    (600, 4, 160, 2, 64, 200),     # three row tiles, 5 and 2 K stages
])
def test_grouped_out_proj(n, n_h, c, g, d_g, d):
    say(f"grouped out proj n={n} n_h={n_h} c={c} g={g} d_g={d_g} d={d}")
    o, WG, WO = synth.out_proj_inputs(n, n_h, c, g, d_g, d, seed=n + d)
    _check_out_proj(o, WG, WO, "small")


def test_grouped_out_proj_flash_shape():
    # the Flash shape (g = 8, d_g = 1024, d = 4096 for 64 heads of 512) over
    # 300 tokens: 64 and 128 K stages, two row tiles
    n = 300
    say(f"grouped out proj Flash shape n={n}")
    o, WG, WO = synth.out_proj_inputs(n, 64, 512, 8, 1024, 4096, seed=61)
    _check_out_proj(o, WG, WO, "flash")


def test_hca_layer_with_norm_and_rope_fp32():
    # HCA with normalised, rotated queries and entries (entry s at m' * s)
    # and the output turned back by -t: the oracle's composed definition with
    # every visible entry selected
    n, mp, nh, nw = 200, 16, 64, 40
    say(f"hca layer with norm and rope, float32 n={n} m'={mp} n_h={nh} n_win={nw}")
    d = synth.hca_inputs(n=n, seed=52, n_h=nh, m_prime=mp)
    d = {k2: (v.float() if isinstance(v, torch.Tensor) and v.dtype == torch.bfloat16 else v) for k2, v in d.items()}
    _, gq = synth.norm_rope_inputs(1, 1, 512, seed=53)
    _, gk = synth.norm_rope_inputs(1, 1, 512, seed=54)
    Cc = torch.tensor(O.compress_pool(to64(d["C"]), to64(d["Z"]), to64(d["B"]), mp), dtype=torch.float32)
    eps, rd, base = 1e-6, 64, 10000.0
    qn = L.csa_norm_rope(g(d["q"]), g(gq), eps, rd, base, 0, 1)
    Cn = L.csa_norm_rope(g(Cc), g(gk), eps, rd, base, 0, mp)
    Rn = L.csa_norm_rope(g(d["kv_raw"]), g(gk), eps, rd, base, 0, 1)
    o = L.hca_attend(qn[None], Cn[None], Rn[None], g(d["sink"]), 0, mp, nw, d["scale"])[0]
    L.csa_norm_rope(o, None, 0.0, rd, base, 0, -1, out=o)
    torch.cuda.synchronize()
    t = np.arange(n)
    vis = [O.visible_entries(int(x), mp) for x in t]
    idx = np.full((n, max(vis)), -1)
    for r, v in enumerate(vis):
        idx[r, :v] = np.arange(v)
    want = O.csa_attend_rope(to64(d["q"]), to64(Cc), idx, to64(d["kv_raw"]), 0, to64(d["sink"]), t, nw,
                             d["scale"], mp, to64(gq), to64(gk), eps, rd, base)
    assert_close(o, want, torch.float32, "hca layer with norm and rope, float32")


def test_hca_attend_norm_rope_fused_prefill():
    # HCA with the query norm and rotation in the attention's Q load and the
    # -t rotation in its epilogue: bf16 queries normalised and rotated, then
    # rounded once, oracle-normalised entries (at m' s) and window rows
    n, mp, nh, nw = 600, 16, 128, 64
    say(f"hca attend with fused query norm and rope, prefill n={n} m'={mp} n_h={nh} n_win={nw}")
    d = synth.hca_inputs(n=n, seed=57, n_h=nh, m_prime=mp)
    _, gq = synth.norm_rope_inputs(1, 1, 512, seed=58)
    _, gk = synth.norm_rope_inputs(1, 1, 512, seed=59)
    eps, rd, base = 1e-6, 64, 10000.0
    st = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)
    t = np.arange(n)
    Cc = O.compress_pool(to64(d["C"]), to64(d["Z"]), to64(d["B"]), mp)
    Cn = st(O.norm_rope(Cc, to64(gk), eps, mp * np.arange(Cc.shape[0]), rd, base))
    Rn = st(O.norm_rope(to64(d["kv_raw"]), to64(gk), eps, t, rd, base))
    out = L.hca_attend_norm_rope(g(d["q"])[None], g(gq), eps, rd, base, g(Cn)[None], g(Rn)[None], g(d["sink"]), 0,
                                 mp, nw, d["scale"])[0]
    torch.cuda.synchronize()
    qn = to64(st(O.norm_rope(to64(d["q"]), to64(gq), eps, t, rd, base)))
    att = O.hca_attend(qn, to64(Cn), to64(Rn), 0, to64(d["sink"]), t, mp, nw, d["scale"])
    assert_close(out, O.rope(att, -t, rd, base), torch.bfloat16, "hca fused norm and rope, prefill")


def test_hca_attend_norm_rope_fused_decode_split():
    # one query per sequence over every completed entry: the list is split
    # over workgroups and each partial output turned back before the merge
    b, n_comp, nw, mp = 2, 3000, 128, 128
    t = n_comp * mp + 9
    eps, rd, base = 1e-6, 64, 10000.0
    say(f"hca attend with fused query norm and rope, decode b={b} n_comp={n_comp} t={t}")
    gen = torch.Generator().manual_seed(71)
    q = (3.0 * torch.randn((b, 1, 64, 512), generator=gen)).to(torch.bfloat16)
    gq = 0.5 + torch.rand(512, generator=gen)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    raw_pos0 = t - nw + 1
    assert L.load_library().hca_attend_workspace_size(b, 1, t, n_comp, 64, 512, mp, nw, 1) > 0
    out = L.hca_attend_norm_rope(g(q), g(gq), eps, rd, base, g(Cc), g(raw), g(sink), t, mp, nw, 1 / math.sqrt(512),
                                 raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    st = lambda a: to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    for s in range(b):
        qn = st(O.norm_rope(to64(q[s]), to64(gq), eps, [t], rd, base))
        att = O.hca_attend(qn, to64(Cc[s]), to64(raw[s]), raw_pos0, to64(sink), [t], mp, nw, 1 / math.sqrt(512))
        assert_close(out[s], O.rope(att, -np.array([t]), rd, base), torch.bfloat16, f"seq {s}")
