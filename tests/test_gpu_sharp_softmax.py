"""GPU parity of the attention kernels' sharp-softmax fallback.

The MFMA attention kernel keeps, per head, a fixed reference maximum taken
from the first tile of entries it reads; when a later logit exceeds that
reference by more than 64 in log2 units the workgroup runs its entries again
with the largest logit as the reference.  These cases use unscaled N(0, 1)
data with softmax scale 1 (logits with a standard deviation of about 23), so
that, as the test checks from the inputs alone, a later tile does exceed the
first one by that much for some heads; the outputs must still match the
oracle: CSA prefill (one workgroup per query), CSA decode (a query's entries
split over several workgroups, then merged), HCA prefill (two queries per
workgroup over the dense entry list) and HCA decode, and the CSA prefill and
decode forms with the query norm and rotation fused in.
"""

import sys

import numpy as np
import pytest
import torch

import long_context_compressed_csa_amd as L
from long_context_compressed_csa_amd import synth
import oracle as O
from parity_helpers import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LOG2E = 1.4426950408889634
HEADROOM = 64.0   # log2 units


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


def _over_headroom(q_t, E, scale, first=16):
    """Heads of one query whose largest logit over the entry list E (in the
    kernel's reading order) exceeds the largest of the first `first` entries
    by more than the headroom (log2 units)."""
    lg = (to64(q_t) @ to64(E).T) * scale * LOG2E
    return int(np.sum(lg.max(axis=1) - lg[:, :first].max(axis=1) > HEADROOM))


def test_csa_prefill_restart():
    n, k, nw, m, scale = 256, 32, 64, 4, 1.0
    say(f"sharp softmax: csa prefill n={n} k={k} n_win={nw} scale={scale}")
    d = synth.prefill_inputs(n=n, seed=61, k=k, unscaled=True)
    Cc = torch.tensor(O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m),
                      dtype=torch.float32).to(torch.bfloat16)
    idx, _ = O.index_topk(to64(d["qI"]), to64(d["w"]), to64(d["KIcomp"]), np.arange(n), m, k)
    # the kernel reads a query's valid selected entries in index order, then its window
    over = 0
    for t in range(0, n, 7):
        sel = idx[t][idx[t] >= 0]
        E = np.concatenate([to64(Cc)[sel], to64(d["kv_raw"])[max(0, t - nw + 1):t + 1]])
        if E.shape[0] > 16:
            over += _over_headroom(d["q"][t], E, scale)
    print(f"[restart] (query, head) pairs past the headroom among sampled queries: {over}", flush=True)
    assert over > 0
    out = L.csa_attend(g(d["q"]), g(Cc), g(torch.tensor(idx, dtype=torch.int32)), g(d["kv_raw"]), g(d["sink"]),
                       0, m, nw, scale)
    torch.cuda.synchronize()
    want = O.csa_attend(to64(d["q"]), to64(Cc), idx, to64(d["kv_raw"]), 0, to64(d["sink"]), np.arange(n), nw,
                        scale, m)
    assert_close(out[0], want, torch.bfloat16, "csa prefill, restarted softmax")


def test_csa_decode_split_restart():
    b, n_comp, k, nw, m, scale = 2, 1500, 512, 128, 4, 1.0
    t = n_comp * m + 1
    say(f"sharp softmax: csa decode b={b} n_comp={n_comp} k={k} scale={scale}")
    gen = torch.Generator().manual_seed(62)
    q = torch.randn((b, 1, 64, 512), generator=gen).to(torch.bfloat16)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    idx = torch.stack([torch.sort(torch.randperm(n_comp, generator=gen)[:k]).values for _ in range(b)])
    idx = idx.to(torch.int32)[:, None, :]
    # plant, in each sequence's second tile, an entry along one query head:
    # its logit (about 2 * 512) dwarfs the first tile's (about 60)
    for s in range(b):
        Cc[s, idx[s, 0, 20]] = (2 * q[s, 0, 5].float()).to(torch.bfloat16)
    raw_pos0 = t - nw + 1
    ws = L.load_library().csa_attend_workspace_size(b, 1, t, n_comp, 64, 512, k, m, nw, 1)
    assert ws > 0, "one query per sequence should split its entries over workgroups"
    # the first split starts with the first 16 selected entries and holds at
    # least the first 32
    over = sum(_over_headroom(q[s, 0], Cc[s, idx[s, 0, :32].long()], scale) for s in range(b))
    print(f"[restart] (sequence, head) pairs past the headroom: {over}", flush=True)
    assert over > 0
    out = L.csa_attend(g(q), g(Cc), g(idx), g(raw), g(sink), t, m, nw, scale, raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    for s in range(b):
        want = O.csa_attend(to64(q[s]), to64(Cc[s]), idx[s].numpy(), to64(raw[s]), raw_pos0, to64(sink), [t], nw,
                            scale, m)
        assert_close(out[s], want, torch.bfloat16, f"csa decode seq {s}, restarted softmax")


def test_hca_prefill_restart():
    n, mp, nw, scale = 512, 8, 64, 1.0
    say(f"sharp softmax: hca prefill n={n} m'={mp} n_win={nw} scale={scale}")
    gen = torch.Generator().manual_seed(63)
    C = torch.randn((n, 512), generator=gen).to(torch.bfloat16)
    Z = torch.randn((n, 512), generator=gen).to(torch.bfloat16)
    B = (0.1 * torch.randn((mp, 512), generator=gen)).to(torch.bfloat16)
    q = torch.randn((n, 64, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    Cc = torch.tensor(O.compress_pool(to64(C), to64(Z), to64(B), mp), dtype=torch.float32).to(torch.bfloat16)
    over = 0
    for t in range(16 * mp, n, 5):
        E = np.concatenate([to64(Cc)[:(t + 1) // mp], to64(C)[max(0, t - nw + 1):t + 1]])
        over += _over_headroom(q[t], E, scale)
    print(f"[restart] (query, head) pairs past the headroom among sampled queries: {over}", flush=True)
    assert over > 0
    out = L.hca_attend(g(q), g(Cc), g(C), g(sink), 0, mp, nw, scale)
    torch.cuda.synchronize()
    want = O.hca_attend(to64(q), to64(Cc), to64(C), 0, to64(sink), np.arange(n), mp, nw, scale)
    assert_close(out[0], want, torch.bfloat16, "hca prefill, restarted softmax")


def test_hca_decode_split_restart():
    b, n_comp, nw, mp, scale = 2, 2000, 128, 128, 1.0
    t = n_comp * mp + 5
    say(f"sharp softmax: hca decode b={b} n_comp={n_comp} scale={scale}")
    gen = torch.Generator().manual_seed(64)
    q = torch.randn((b, 1, 64, 512), generator=gen).to(torch.bfloat16)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    for s in range(b):
        Cc[s, 20] = (2 * q[s, 0, 5].float()).to(torch.bfloat16)
    raw_pos0 = t - nw + 1
    ws = L.load_library().hca_attend_workspace_size(b, 1, t, n_comp, 64, 512, mp, nw, 1)
    assert ws > 0, "one query per sequence should split its entries over workgroups"
    over = sum(_over_headroom(q[s, 0], Cc[s, :32], scale) for s in range(b))
    print(f"[restart] (sequence, head) pairs past the headroom: {over}", flush=True)
    assert over > 0
    out = L.hca_attend(g(q), g(Cc), g(raw), g(sink), t, mp, nw, scale, raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    for s in range(b):
        want = O.hca_attend(to64(q[s]), to64(Cc[s]), to64(raw[s]), raw_pos0, to64(sink), [t], mp, nw, scale)
        assert_close(out[s], want, torch.bfloat16, f"hca decode seq {s}, restarted softmax")


def _st(a):
    return to64(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))


def test_csa_prefill_restart_fused_norm_rope():
    # the same fallback behind the fused query norm: queries of random signs,
    # unit gain, eps 0 and no rotation, so that the normalised query is the
    # raw one exactly on both sides (with logits this sharp a one-step bf16
    # rounding difference of a query element between the float32 kernel and
    # the float64 oracle would decide near-ties); the decode case below
    # covers the rotation under the fallback
    n, k, nw, m, scale = 256, 32, 64, 4, 1.0
    eps, rd, base = 0.0, 0, 10000.0
    say(f"sharp softmax: csa prefill with fused norm n={n} k={k} n_win={nw} scale={scale}")
    d = synth.prefill_inputs(n=n, seed=65, k=k, unscaled=True)
    q = torch.sign(d["q"].float()).where(d["q"] != 0, torch.ones(())).to(torch.bfloat16)
    gq = torch.ones(512)
    Cc = torch.tensor(O.compress_overlap(*(to64(d[x]) for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m),
                      dtype=torch.float32).to(torch.bfloat16)
    idx, _ = O.index_topk(to64(d["qI"]), to64(d["w"]), to64(d["KIcomp"]), np.arange(n), m, k)
    t_pos = np.arange(n)
    qn = O.norm_rope(to64(q), to64(gq), eps, t_pos, rd, base)
    assert np.array_equal(qn, to64(q)), "the normalised query is the raw one"
    over = 0
    for t in range(0, n, 7):
        sel = idx[t][idx[t] >= 0]
        E = np.concatenate([to64(Cc)[sel], to64(d["kv_raw"])[max(0, t - nw + 1):t + 1]])
        if E.shape[0] > 16:
            over += _over_headroom(qn[t], E, scale)
    print(f"[restart] (query, head) pairs past the headroom among sampled queries: {over}", flush=True)
    assert over > 0
    out = L.csa_attend_norm_rope(g(q)[None], g(gq), eps, rd, base, g(Cc)[None],
                                 g(torch.tensor(idx, dtype=torch.int32))[None], g(d["kv_raw"])[None], g(d["sink"]),
                                 0, m, nw, scale)
    torch.cuda.synchronize()
    want = O.csa_attend(qn, to64(Cc), idx, to64(d["kv_raw"]), 0, to64(d["sink"]), t_pos, nw, scale, m)
    assert_close(out[0], want, torch.bfloat16, "fused csa prefill, restarted softmax")


def test_csa_decode_split_restart_fused_norm_rope():
    b, n_comp, k, nw, m, scale = 2, 1500, 512, 128, 4, 1.0
    eps, rd, base = 1e-6, 64, 10000.0
    t = n_comp * m + 1
    say(f"sharp softmax: csa decode with fused norm and rope b={b} n_comp={n_comp} k={k} scale={scale}")
    gen = torch.Generator().manual_seed(67)
    q = (2.0 * torch.randn((b, 1, 64, 512), generator=gen)).to(torch.bfloat16)
    gq = 1.0 + 0.1 * torch.randn(512, generator=gen)
    Cc = torch.randn((b, n_comp, 512), generator=gen).to(torch.bfloat16)
    raw = torch.randn((b, nw, 512), generator=gen).to(torch.bfloat16)
    sink = torch.randn(64, generator=gen)
    idx = torch.stack([torch.sort(torch.randperm(n_comp, generator=gen)[:k]).values for _ in range(b)])
    idx = idx.to(torch.int32)[:, None, :]
    qn = [_st(O.norm_rope(to64(q[s]), to64(gq), eps, [t], rd, base)) for s in range(b)]
    # plant, in each sequence's second tile, an entry along one normalised head
    for s in range(b):
        Cc[s, idx[s, 0, 20]] = torch.tensor(2 * qn[s][0, 5], dtype=torch.float32).to(torch.bfloat16)
    raw_pos0 = t - nw + 1
    over = sum(_over_headroom(qn[s][0], Cc[s, idx[s, 0, :32].long()], scale) for s in range(b))
    print(f"[restart] (sequence, head) pairs past the headroom: {over}", flush=True)
    assert over > 0
    out = L.csa_attend_norm_rope(g(q), g(gq), eps, rd, base, g(Cc), g(idx), g(raw), g(sink), t, m, nw, scale,
                                 raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    for s in range(b):
        att = O.csa_attend(qn[s], to64(Cc[s]), idx[s].numpy(), to64(raw[s]), raw_pos0, to64(sink), [t], nw, scale, m)
        assert_close(out[s], O.rope(att, -np.array([t]), rd, base), torch.bfloat16,
                     f"fused csa decode seq {s}, restarted softmax")
