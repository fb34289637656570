"""csa_index_topk_noalloc (the index + top-k entry point that takes no
workspace: its scratch is the library's per-GPU device array) against
csa_index_topk with a caller workspace, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, so the
second runs on scratch the first left dirty: the selections and scores must
be bit-identical to the workspace entry point's (integer work, and the same
kernels in the same order).  Shapes cover the decode path (streaming scorer,
threshold filter and merge), the multi-stage general selection and the fused
prefill scorer.
"""

import math
import sys

import pytest
import torch

import long_context_compressed_csa_amd as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(seed, b, n_q, n_comp, nh=64, cI=128, dtype=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    qI = (torch.randn((b, n_q, nh, cI), generator=gen) / math.sqrt(cI)).to(dtype)
    w = torch.nn.functional.softplus(torch.randn((b, n_q, nh), generator=gen))
    KI = (torch.randn((b, n_comp, cI), generator=gen) / math.sqrt(cI)).to(dtype)
    return qI.to(DEV), w.to(DEV), KI.to(DEV)


CASES = [
    # (name, b, n_q, n_comp, k, m): the first of each pair is the larger
    ("decode, threshold path", 4, 1, 60000, 512, 4),
    ("decode, smaller", 2, 1, 9000, 128, 4),
    ("general multi-stage path", 1, 5, 20000, 256, 4),
    ("general, smaller", 1, 3, 5000, 64, 4),
    ("prefill, fused selection", 1, 1024, 256, 64, 4),
    ("prefill, smaller", 1, 256, 64, 16, 4),
]


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3), (4, 5), (0, 5)])
def test_noalloc_matches_workspace_entry_point(first, second):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    lib = L.load_library()
    for ci in (first, second):
        name, b, n_q, n_comp, k, m = CASES[ci]
        t0 = max(0, n_comp * m - n_q)   # the last query sees all n_comp entries
        say(f"noalloc {name}: b={b} n_q={n_q} n_comp={n_comp} k={k} t0={t0}")
        need = lib.csa_index_topk_workspace_size(b, n_q, n_comp, k)
        assert 0 < need <= 80 * 1024 * 1024
        qI, w, KI = _inputs(100 + ci, b, n_q, n_comp)
        want_i, want_s = L.csa_index_topk(qI, w, KI, t0, m, k, score=True)
        got_i, got_s = L.csa_index_topk_noalloc(qI, w, KI, t0, m, k, score=True)
        torch.cuda.synchronize()
        assert torch.equal(got_i, want_i), f"{name}: selections differ"
        assert torch.equal(got_s, want_s), f"{name}: scores differ"
        # every query with a visible entry selected something
        vis = (t0 + torch.arange(n_q, device=DEV) + 1) // m
        assert (got_i[..., 0][:, vis > 0] >= 0).all()
