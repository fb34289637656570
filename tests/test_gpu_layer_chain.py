"""The bf16 CSA prefill layer as the benchmark runs it, chained on the GPU,
against the oracle computed from the same inputs alone.

GPU chain (n = 8192, 64 heads, c = 512, m = 4, k = 512, n_win = 128,
indexer 64 x 128): the overlapped compressor on the main streams and on the
indexer-key streams, then scoring with fused top-k on the GPU's own keys,
then attention on the GPU's own entries and selection.

Oracle chain: both compressors in float64, stored in bf16 (round to nearest
even: the storage the bf16 layer keeps between its steps), then scores,
top-k and attention in float64 on those entries.  Compared on sampled
queries that cover the first positions, both sides of the entry boundary at
2048 and the last positions: compressed entries and keys element-wise;
index sets bit-exact apart from near-ties; the chained attention output
where the GPU chose the oracle's set; and on every sampled query the GPU
attention step run on the oracle's selection.
"""

import sys

import numpy as np
import pytest
import torch

import long_context_compressed_csa_amd as L
from long_context_compressed_csa_amd import synth
import oracle as O
from parity_helpers import assert_close, assert_index_sets, to64

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


def _bf16(a):
    return to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))


def test_csa_prefill_layer_chained_bf16():
    say("chained bf16 CSA prefill layer, n=8192 (sampled queries)")
    d = synth.prefill_inputs(device=DEV)
    p = d["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    Cc = L.csa_compress(*(d[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    KI = L.csa_compress(*(d[x] for x in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")), m)
    idx = L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k)
    out = L.csa_attend(d["q"], Cc, idx, d["kv_raw"], d["sink"], 0, m, nw, d["scale"])
    torch.cuda.synchronize()

    Cc_o = O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    KI_o = O.compress_overlap(*(to64(d[x]) for x in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")), m)
    assert_close(Cc, Cc_o, torch.bfloat16, "compressed entries")
    assert_close(KI, KI_o, torch.bfloat16, "compressed indexer keys")
    Cc16, KI16 = _bf16(Cc_o), _bf16(KI_o)

    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(2040, 2057), np.arange(n - 8, n),
                                     np.random.default_rng(5).integers(0, n, 16)]))
    sc = O.index_scores(to64(d["qI"][rows]), to64(d["w"][rows]), KI16, rows, m)
    vis = np.minimum((rows + 1) // m, n // m)
    oi = np.stack([O.topk_select(sc[r], int(vis[r]), k) for r in range(len(rows))])
    gi = idx[0, rows].cpu().numpy()
    n_ties = assert_index_sets(gi, oi, sc, vis, k, "chained selection")
    print(f"[ties] {n_ties} of {len(rows)} sampled queries settled a near-tie differently", flush=True)
    assert n_ties <= len(rows) // 4

    want = O.csa_attend(to64(d["q"][rows]), Cc16, oi, to64(d["kv_raw"]), 0, to64(d["sink"]), rows, nw,
                        d["scale"], m)
    same = np.array([set(gi[r].tolist()) == set(oi[r].tolist()) for r in range(len(rows))])
    assert_close(out[0, rows[same]], want[same], torch.bfloat16, "chained attention output")
    # the attention step on the oracle's selection for every sampled query
    # (the other rows keep the GPU's selection: any valid input)
    idx_o = idx.clone()
    idx_o[0, rows] = torch.tensor(oi, dtype=torch.int32, device=DEV)
    out_o = L.csa_attend(d["q"], Cc, idx_o, d["kv_raw"], d["sink"], 0, m, nw, d["scale"])
    torch.cuda.synchronize()
    assert_close(out_o[0, rows], want, torch.bfloat16, "attention on the oracle's selection")
