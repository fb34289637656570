"""Comparison rules shared by the GPU parity tests.

Floats: RMS is taken per output vector (one attention output o[t, h, :] or
one compressed entry C[i, :], the last axis), so that rows of very different
scale -- a query reading 3 entries next to one reading 600 -- are each held
to their own scale.  Then |got - want| <= 2e-2 * RMS + 2^-8 * |want|
element-wise for bfloat16 storage (the stated bound plus half a bfloat16 ulp
of the element itself: storing a result in bfloat16 alone moves it by up to
2^-8 of its magnitude, which exceeds 2e-2 * RMS for elements above
5.12 * RMS), and |got - want| <= 1e-4 * min(1, RMS) for float32.  Index sets: equal, except that a
member of the symmetric difference may lie within 1e-3 of the k-th oracle
score (a near-tie decided differently by float32 and float64 sums); sizes,
ascending order and -1 padding must match exactly.
"""

import numpy as np
import torch

BF16_TOL = 2e-2
F32_TOL = 1e-4
BF16_HALF_ULP = 2.0 ** -8
TIE_TOL = 1e-3


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def assert_close(got, want, dtype, what=""):
    got, want = to64(got), to64(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if not want.size:
        return 0.0, 0.0
    rms = np.sqrt(np.mean(want ** 2, axis=-1, keepdims=True))
    diff = np.abs(got - want)
    if dtype == torch.bfloat16:
        bound = BF16_TOL * rms + BF16_HALF_ULP * np.abs(want)
    else:
        bound = F32_TOL * np.minimum(1.0, rms) + 0.0 * want
    excess = diff - bound
    i = int(np.argmax(excess))
    idx = np.unravel_index(i, want.shape)
    row_rms = float(rms[idx[:-1] + (0,)])
    assert excess.flat[i] <= 0, (f"{what}: |err| {diff.flat[i]:.3e} > bound {bound.flat[i]:.3e} at "
                                 f"{idx} (want {want.flat[i]:.4e}, row rms {row_rms:.3e})")
    return float(diff.max()), float(np.sqrt(np.mean(want ** 2)))


def assert_index_sets(got_idx, want_idx, oracle_scores, vis, k, what=""):
    """got_idx/want_idx [n_q, k]; oracle_scores [n_q, >=max vis]; vis [n_q]."""
    got_idx = np.asarray(got_idx)
    want_idx = np.asarray(want_idx)
    n_ties = 0
    for r in range(got_idx.shape[0]):
        take = min(k, int(vis[r]))
        g, w = got_idx[r], want_idx[r]
        assert np.all(g[take:] == -1) and np.all(w[take:] == -1), (what, r, "padding")
        gv, wv = g[:take], w[:take]
        assert np.all(np.diff(gv) > 0), (what, r, "not strictly ascending")
        assert gv.min(initial=0) >= 0 and (take == 0 or gv.max() < vis[r]), (what, r, "invisible index")
        diff = set(gv.tolist()) ^ set(wv.tolist())
        if diff:
            kth = np.sort(oracle_scores[r, : int(vis[r])])[::-1][take - 1]
            for s in diff:
                assert abs(oracle_scores[r, s] - kth) <= TIE_TOL, (what, r, s, oracle_scores[r, s], kth)
            n_ties += 1
    return n_ties
