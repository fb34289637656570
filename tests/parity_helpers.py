"""Comparison rules shared by the GPU parity tests.

Floats: RMS is taken per output vector (one attention output o[t, h, :] or
one compressed entry C[i, :], the last axis), so that rows of very different
scale -- a query reading 3 entries next to one reading 600 -- are each held
to their own scale.  Then |got - want| <= max(2e-2 * RMS, ulp(want))
element-wise for bfloat16 storage, where ulp(x) = 2^(floor(log2 |x|) - 7) is
the spacing of bfloat16 values at x: the stated bound, except for elements
above 2.56 * RMS, where one bfloat16 step is larger than 2e-2 * RMS and the
stored result must be within one step of the exact one (bfloat16 cannot
resolve the stated bound there); and |got - want| <= 1e-4 * min(1, RMS) for
float32.  Every comparison prints its
worst error as a fraction of its bound and of the plain 2e-2 * RMS (1e-4 *
min(1, RMS)) bound, so the margin is on record.  Index sets: equal, except that a
member of the symmetric difference may lie within 1e-3 of the k-th oracle
score (a near-tie decided differently by float32 and float64 sums); sizes,
ascending order and -1 padding must match exactly.
"""

import numpy as np
import torch

BF16_TOL = 2e-2
F32_TOL = 1e-4


def bf16_ulp(x):
    """Spacing of bfloat16 values at x (8 significant bits): 2^(e - 7) for
    2^e <= |x| < 2^(e+1); 0 at x = 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)

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
        plain = BF16_TOL * rms + 0.0 * want
        bound = np.maximum(plain, bf16_ulp(want))
    else:
        plain = F32_TOL * np.minimum(1.0, rms) + 0.0 * want
        bound = plain
    # a zero bound (an all-zero oracle row) demands an exact zero
    ratio = np.where(bound > 0, diff / np.where(bound > 0, bound, 1.0), np.where(diff > 0, np.inf, 0.0))
    plain_ratio = np.where(plain > 0, diff / np.where(plain > 0, plain, 1.0), np.where(diff > 0, np.inf, 0.0))
    i = int(np.argmax(ratio))
    idx = np.unravel_index(i, want.shape)
    row_rms = float(rms[idx[:-1] + (0,)])
    print(f"[margin] {what or 'output'}: worst err/bound {ratio.flat[i]:.3f}, "
          f"worst err/plain bound {float(plain_ratio.max()):.3f}", flush=True)
    assert ratio.flat[i] <= 1.0, (f"{what}: |err| {diff.flat[i]:.3e} > bound {bound.flat[i]:.3e} at "
                                  f"{idx} (want {want.flat[i]:.4e}, row rms {row_rms:.3e})")
    return float(diff.max()), float(np.sqrt(np.mean(want ** 2)))


def assert_index_sets(got_idx, want_idx, oracle_scores, vis, k, what="", tie_tol=TIE_TOL):
    """got_idx/want_idx [n_q, k]; oracle_scores [n_q, >=max vis]; vis [n_q].
    tie_tol: how far from the k-th oracle score a member of the symmetric
    difference may lie (1e-3 for float32 scores)."""
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
                assert abs(oracle_scores[r, s] - kth) <= tie_tol, (what, r, s, oracle_scores[r, s], kth)
            n_ties += 1
    return n_ties
