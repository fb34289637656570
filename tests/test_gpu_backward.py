"""GPU parity of the backward pass (attention and compressors) against the
oracle's gradients, which are pinned to central differences and torch
autograd on the CPU.  Gradients are float32 on the GPU; they are held to the
float32 bound (1e-4 * min(1, RMS) per row), also for bf16 inputs, whose
values the oracle receives exactly.  The reductions are deterministic: a
repeated call gives bit-identical gradients, and a sequence processed as two
query blocks (accumulating) gives the whole sequence's gradients.
"""

import math
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


def _check_grads(got, want, what):
    dq, dC, dR, ds = got
    wq, wC, wR, ws = want
    assert_close(dq, wq, torch.float32, f"{what}: dq")
    assert_close(dC, wC, torch.float32, f"{what}: dCcomp")
    assert_close(dR, wR, torch.float32, f"{what}: dkv_raw")
    assert_close(ds[None], ws[None], torch.float32, f"{what}: dsink")


def _csa_case(n, nh, c, k, nw, m, dtype, seed, unscaled=True):
    gen = torch.Generator().manual_seed(seed)
    sd = 1.0 if unscaled else 1.0 / math.sqrt(c)
    q = (torch.randn((n, nh, c), generator=gen) * sd).to(dtype)
    Cc = (torch.randn((n // m, c), generator=gen) * sd).to(dtype)
    raw = (torch.randn((n, c), generator=gen) * sd).to(dtype)
    sink = torch.randn(nh, generator=gen)
    dout = torch.randn((n, nh, c), generator=gen).to(dtype)
    idx = np.stack([O.topk_select(np.random.default_rng(seed * 1000 + t).normal(size=n // m),
                                  O.visible_entries(t, m), k) for t in range(n)]).astype(np.int32)
    return q, Cc, raw, sink, dout, idx


@pytest.mark.parametrize("n,nh,c,k,nw,m,dtype", [
    (64, 4, 32, 4, 16, 4, torch.float32),      # the tiny layer's shape
    (96, 3, 40, 7, 9, 4, torch.float32),       # ragged slot tiles, odd sizes
    (256, 64, 512, 32, 64, 4, torch.bfloat16), # the layer's head shape
    (72, 128, 512, 8, 16, 4, torch.bfloat16),  # two head groups (per-query step on MFMA, contributions not)
])
def test_csa_attend_backward(n, nh, c, k, nw, m, dtype):
    say(f"csa attend backward n={n} n_h={nh} c={c} k={k} n_win={nw} {dtype}")
    q, Cc, raw, sink, dout, idx = _csa_case(n, nh, c, k, nw, m, dtype, seed=n + c)
    scale = 1.0 / math.sqrt(c)
    got = L.csa_attend_backward(g(q), g(Cc), g(torch.tensor(idx)), g(raw), g(sink), g(dout), 0, m, nw, scale)
    torch.cuda.synchronize()
    want = O.csa_attend_backward(to64(q), to64(Cc), idx, to64(raw), 0, to64(sink), np.arange(n), nw, scale,
                                 to64(dout), m)
    _check_grads([x[0] if x.dim() > 1 and x.shape[0] == 1 else x for x in got], want, "csa")


def test_csa_attend_backward_deterministic_and_blockwise():
    n, nh, c, k, nw, m = 200, 64, 512, 16, 32, 4
    say(f"csa attend backward determinism and query blocks n={n}")
    q, Cc, raw, sink, dout, idx = _csa_case(n, nh, c, k, nw, m, torch.bfloat16, seed=7)
    scale = 1.0 / math.sqrt(c)
    args = (g(q), g(Cc), g(torch.tensor(idx)), g(raw), g(sink), g(dout), 0, m, nw, scale)
    a = [x.clone() for x in L.csa_attend_backward(*args)]
    b = L.csa_attend_backward(*args)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "repeated backward differs"
    # two query blocks, the second accumulating into the entry, row and sink gradients
    h = 120
    f = dict(dtype=torch.float32, device=DEV)
    grads = (torch.empty((1, h, nh, c), **f), torch.zeros((1, n // m, c), **f), torch.zeros((1, n, c), **f),
             torch.zeros(nh, **f))
    L.csa_attend_backward(g(q[:h]), g(Cc), g(torch.tensor(idx[:h])), g(raw), g(sink), g(dout[:h]), 0, m, nw, scale,
                          grads=grads)
    dq1 = grads[0].clone()
    grads2 = (torch.empty((1, n - h, nh, c), **f), grads[1], grads[2], grads[3])
    L.csa_attend_backward(g(q[h:]), g(Cc), g(torch.tensor(idx[h:])), g(raw), g(sink), g(dout[h:]), h, m, nw, scale,
                          accumulate=True, grads=grads2)
    torch.cuda.synchronize()
    want = O.csa_attend_backward(to64(q), to64(Cc), idx, to64(raw), 0, to64(sink), np.arange(n), nw, scale,
                                 to64(dout), m)
    _check_grads([torch.cat([dq1[0], grads2[0][0]]), grads[1][0], grads[2][0], grads[3]], want, "two blocks")


@pytest.mark.parametrize("n,mp,nw,nh,c,dtype", [
    (80, 8, 12, 4, 32, torch.float32),
    (300, 16, 64, 64, 512, torch.bfloat16),
])
def test_hca_attend_backward(n, mp, nw, nh, c, dtype):
    say(f"hca attend backward n={n} m'={mp} n_win={nw} n_h={nh} c={c} {dtype}")
    gen = torch.Generator().manual_seed(n)
    q = torch.randn((n, nh, c), generator=gen).to(dtype)
    Cc = torch.randn((n // mp, c), generator=gen).to(dtype)
    raw = torch.randn((n, c), generator=gen).to(dtype)
    sink = torch.randn(nh, generator=gen)
    dout = torch.randn((n, nh, c), generator=gen).to(dtype)
    scale = 1.0 / math.sqrt(c)
    got = L.hca_attend_backward(g(q), g(Cc), g(raw), g(sink), g(dout), 0, mp, nw, scale)
    torch.cuda.synchronize()
    want = O.hca_attend_backward(to64(q), to64(Cc), to64(raw), 0, to64(sink), np.arange(n), mp, nw, scale, to64(dout))
    _check_grads([x[0] if x.dim() > 1 and x.shape[0] == 1 else x for x in got], want, "hca")


@pytest.mark.parametrize("dtype,n,c,m,b,prev,overlap", [
    (torch.float32, 38, 24, 4, 2, False, True),    # ragged tail, batch of 2
    (torch.float32, 40, 16, 4, 1, True, True),     # continuing from a previous block
    (torch.bfloat16, 1024, 512, 4, 1, False, True),
    (torch.bfloat16, 1030, 512, 4, 2, True, True),  # bias sums in the row kernel: batch, state, ragged tail
    (torch.bfloat16, 200, 64, 4, 3, True, True),    # eight dimension groups per row
    (torch.float32, 300, 16, 32, 1, False, False), # pooling, ragged tail
    (torch.bfloat16, 4096, 512, 128, 1, False, False),
])
def test_compress_backward(dtype, n, c, m, b, prev, overlap):
    say(f"compress backward {dtype} n={n} c={c} m={m} b={b} prev={prev} overlap={overlap}")
    gen = torch.Generator().manual_seed(n + m)
    rnd = lambda *s, sd=1.0: (torch.randn(s, generator=gen) * sd).to(dtype)
    Ca, Za = rnd(b, n, c), rnd(b, n, c, sd=2.0)
    Ba = rnd(m, c, sd=0.3)
    Cb, Zb, Bb = (rnd(b, n, c), rnd(b, n, c, sd=2.0), rnd(m, c, sd=0.3)) if overlap else (None, None, None)
    pC, pZ = (rnd(b, m, c), rnd(b, m, c, sd=2.0)) if prev else (None, None)
    dCc = torch.randn((b, n // m, c), generator=gen)
    G = lambda x: None if x is None else g(x)
    got = L.csa_compress_backward(G(Ca), G(Cb), G(Za), G(Zb), G(Ba), G(Bb), m, g(dCc), prev_Cb=G(pC), prev_Zb=G(pZ),
                                  overlap=overlap)
    torch.cuda.synchronize()
    want_b = {k: 0.0 for k in ("dBa", "dBb")}
    for s in range(b):
        if overlap:
            w = O.compress_overlap_backward(to64(Ca[s]), to64(Cb[s]), to64(Za[s]), to64(Zb[s]), to64(Ba), to64(Bb), m,
                                            to64(dCc[s]), None if pC is None else to64(pC[s]),
                                            None if pZ is None else to64(pZ[s]))
        else:
            w = O.compress_pool_backward(to64(Ca[s]), to64(Za[s]), to64(Ba), m, to64(dCc[s]))
            w = {"dCa": w["dC"], "dZa": w["dZ"], "dBa": w["dB"]}
        for key in ("dCa", "dZa") + (("dCb", "dZb") if overlap else ()):
            assert_close(got[key][s], w[key], torch.float32, f"{key} seq {s}")
        if prev:
            assert_close(got["dprev_Cb"][s], w["dprev_Cb"], torch.float32, "dprev_Cb")
            assert_close(got["dprev_Zb"][s], w["dprev_Zb"], torch.float32, "dprev_Zb")
        for key in ("dBa",) + (("dBb",) if overlap else ()):
            want_b[key] = want_b[key] + w[key]
    for key in ("dBa",) + (("dBb",) if overlap else ()):
        assert_close(got[key], want_b[key], torch.float32, key)
