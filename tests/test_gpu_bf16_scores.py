"""GPU parity of the BF16 index-score option (CSA_SCORE_BF16): the selection
runs on scores rounded to bfloat16.  The oracle rounds its float64 scores the
same way (torch's round to nearest even) and selects with the same tie rule,
so the index sets must agree except where a float32 and a float64 score
round to neighbouring bfloat16 values: a member of the symmetric difference
may then lie one bfloat16 step from the k-th rounded score.  The recall of
the rounded selection against the float32 one is printed."""

import math
import sys

import numpy as np
import pytest
import torch

import long_context_compressed_csa_amd as L
from long_context_compressed_csa_amd import synth
import oracle as O
from parity_helpers import assert_index_sets, bf16_ulp, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _round_bf16(x):
    return to64(torch.tensor(x, dtype=torch.float64).to(torch.bfloat16))


def _check(qI, w, KI, t_pos, m, k, got, what):
    sc = O.index_scores(to64(qI), to64(w), to64(KI), t_pos, m)
    scb = np.where(np.isfinite(sc), _round_bf16(np.where(np.isfinite(sc), sc, 0.0)), sc)
    n_comp = KI.shape[0]
    vis = [min((int(t) + 1) // m, n_comp) for t in t_pos]
    want = np.stack([O.topk_select(scb[r], vis[r], k) for r in range(len(t_pos))])
    kth = np.array([np.sort(scb[r, :vis[r]])[::-1][min(k, vis[r]) - 1] if vis[r] else 1.0 for r in range(len(t_pos))])
    tol = float(bf16_ulp(np.abs(kth)).max())
    ties = assert_index_sets(got, want, scb, vis, k, what, tie_tol=tol)
    print(f"[ties] {what}: {ties} of {len(t_pos)} rows settled a boundary differently", flush=True)


def _recall(a, b):
    """Mean over rows of |set(a) & set(b)| / |set(a)| (valid entries)."""
    rs = []
    for x, y in zip(a, b):
        x, y = set(x[x >= 0].tolist()), set(y[y >= 0].tolist())
        if x:
            rs.append(len(x & y) / len(x))
    return float(np.mean(rs))


def test_bf16_scores_prefill_fused():
    n, m, k = 1024, 4, 64
    say(f"bf16 index scores, prefill n={n} k={k}")
    d = synth.prefill_inputs(n=n, seed=81, k=k)
    idx32 = L.csa_index_topk(d["qI"].to(DEV), d["w"].to(DEV), d["KIcomp"].to(DEV), 0, m, k)
    idx16 = L.csa_index_topk(d["qI"].to(DEV), d["w"].to(DEV), d["KIcomp"].to(DEV), 0, m, k, bf16_scores=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(n - 8, n), np.random.default_rng(8).integers(0, n, 48)]))
    _check(d["qI"][rows], d["w"][rows], d["KIcomp"], rows, m, k, idx16[0, rows].cpu().numpy(), "prefill")
    print(f"[recall] prefill bf16 vs float32 scores: {_recall(idx32[0].cpu().numpy(), idx16[0].cpu().numpy()):.4f}",
          flush=True)


def test_bf16_scores_decode_stream():
    b, n_comp, k, m = 4, 40000, 512, 4
    t = n_comp * m + 1
    say(f"bf16 index scores, decode b={b} n_comp={n_comp} k={k}")
    gen = torch.Generator().manual_seed(82)
    qI = (torch.randn((b, 1, 64, 128), generator=gen) / math.sqrt(128)).to(torch.bfloat16)
    w = torch.nn.functional.softplus(torch.randn((b, 1, 64), generator=gen))
    KI = (torch.randn((b, n_comp, 128), generator=gen) / math.sqrt(128)).to(torch.bfloat16)
    idx32 = L.csa_index_topk(qI.to(DEV), w.to(DEV), KI.to(DEV), t, m, k)
    idx16 = L.csa_index_topk(qI.to(DEV), w.to(DEV), KI.to(DEV), t, m, k, bf16_scores=True)
    torch.cuda.synchronize()
    for s in range(b):
        _check(qI[s], w[s], KI[s], [t], m, k, idx16[s].cpu().numpy(), f"decode seq {s}")
    print(f"[recall] decode bf16 vs float32 scores: "
          f"{_recall(idx32[:, 0].cpu().numpy(), idx16[:, 0].cpu().numpy()):.4f}", flush=True)
