"""Seeded synthetic inputs at the shapes of the CSA / HCA workloads.

This module only draws random numbers (and rounds them to the storage
dtype); it contains none of the method's arithmetic.  The test suite feeds
the same tensors to the HIP library and to the CPU oracle.

Recipes (all Gaussian; "scaled" means N(0,1) / sqrt(last dim)):

  tiny      n=64, c=32, m=4, n_h=4, k=4, n_win=16, indexer 2 heads x 16,
            float32, seed 0.  Ca, Cb, Za, Zb, q, qI, KIcomp ~ N(0,1);
            w = softplus(N(0,1)); Ba, Bb ~ N(0, 0.1^2); sink ~ N(0,1).
  compress  n=65536, c=512, bf16.  Overlapped m=4: Ca, Cb ~ N(0,1),
            Za, Zb ~ N(0, 2^2), Ba, Bb ~ N(0, 0.1^2).  Pooling m'=128:
            C ~ N(0,1), Z ~ N(0, 2^2), B ~ N(0, 0.1^2).
  prefill   n=8192, n_h=64, c=512, m=4, k=512, n_win=128, indexer 64 x 128,
            bf16; every tensor scaled, w = softplus(N(0,1)), sink ~ N(0,1).
            The indexer-key streams ICa..IZb [n, 128] (scaled) feed the
            indexer-key compressor; KIcomp [n/4, 128] is also drawn directly
            for stage tests.
  hca       n=131072, m'=128, n_h=64, c=512, n_win=128, bf16; C, Z, q, B
            scaled; sink ~ N(0,1).
  decode    8 sequences with 1,048,576 tokens of history: Ccomp
            [8, 262144, 512] and KIcomp [8, 262144, 128] scaled, window
            [8, 128, 512], previous-block state (Cb, Zb, ICb, IZb, 4 rows
            each), and per step one new token per sequence (Ca..IZb rows),
            q [8, 1, 64, 512], qI [8, 1, 64, 128], w, sink.

"N(mu, x)" is read with x the standard deviation.  Large tensors can be drawn
on the GPU with a seeded device generator; the draw order is fixed.
"""

from __future__ import annotations

import math

import torch

TINY = dict(n=64, c=32, m=4, n_h=4, k=4, n_win=16, n_hI=2, c_I=16, dtype=torch.float32, seed=0)
COMPRESS = dict(n=65536, c=512, m=4, m_prime=128, dtype=torch.bfloat16, seed=2)
PREFILL = dict(n=8192, n_h=64, c=512, m=4, k=512, n_win=128, n_hI=64, c_I=128,
               dtype=torch.bfloat16, seed=3)
HCA = dict(n=131072, m_prime=128, n_h=64, c=512, n_win=128, dtype=torch.bfloat16, seed=4)
DECODE = dict(b=8, history=1 << 20, m=4, n_h=64, c=512, k=512, n_win=128, n_hI=64, c_I=128,
              steps=4, dtype=torch.bfloat16, seed=5)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, g, std=1.0, dtype=torch.float32, device="cpu"):
    """N(0, std^2) drawn in float32, then stored as `dtype`."""
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def scaled(shape, g, dtype, device="cpu"):
    """N(0,1) / sqrt(last dim)."""
    return normal(shape, g, 1.0 / math.sqrt(shape[-1]), dtype, device)


def softplus_normal(shape, g, device="cpu"):
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return torch.nn.functional.softplus(x)


def to_fp8(x):
    """Round a tensor to 8-bit E4M3 codes (torch.float8_e4m3fn, nearest
    even); the draws here stay far inside its +-448 range."""
    return x.float().to(torch.float8_e4m3fn)


def hca_decode_inputs(device="cpu", seed=9):
    """HCA attention state at the 1M-context decode shape: 8 sequences, each
    with 2^20 / 128 = 8192 completed HCA entries and a 128-row window, one
    query per sequence; entries, window and queries N(0,1)/sqrt(c), sink
    logits N(0,1)."""
    p = dict(b=8, n_comp=8192, c=512, n_h=64, m_prime=128, n_win=128, t=(1 << 20) + 3)
    g = _gen(seed, device)
    b, ne, c, nh, nw = p["b"], p["n_comp"], p["c"], p["n_h"], p["n_win"]
    return {"params": p,
            "Ccomp": scaled((b, ne, c), g, torch.bfloat16, device),
            "window": scaled((b, nw, c), g, torch.bfloat16, device),
            "q": scaled((b, 1, nh, c), g, torch.bfloat16, device),
            "sink": normal((nh,), g, 1.0, torch.float32, device)}


def to_mxfp4(x):
    """Round a tensor to OCP MXFP4 along its last dimension (a multiple of
    32): returns (codes, scales), uint8 tensors [..., c / 2] and [..., c / 32].
    Each block of 32 takes the E8M0 scale 2^(floor(log2 max|x|) - 2) (the
    largest E2M1 magnitude is 6 = 1.5 * 2^2); every element divided by it is
    rounded to the nearest E2M1 value (the smaller magnitude on a tie) and
    saturated at 6.  Byte j of a row holds element 2j in its low nibble and
    element 2j + 1 in its high nibble.  An all-zero block gets scale 2^-127."""
    x = x.float()
    *lead, c = x.shape
    assert c % 32 == 0, "MXFP4 blocks are 32 elements"
    blk = x.reshape(*lead, c // 32, 32)
    amax = blk.abs().amax(dim=-1, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    y = (blk / torch.exp2(e)).abs()
    mags = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device=x.device)
    mids = (mags[1:] + mags[:-1]) / 2
    code = torch.bucketize(y, mids)            # nearest magnitude (ties to the smaller)
    code = code | torch.where(blk < 0, 8, 0)   # sign bit
    code = code.reshape(*lead, c).to(torch.uint8)
    codes = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    scales = (e.squeeze(-1) + 127).to(torch.uint8)
    return codes, scales


def tiny_inputs(seed=None, n=None):
    """The tiny float32 CSA layer."""
    p = dict(TINY)
    if n is not None:
        p["n"] = n
    g = _gen(p["seed"] if seed is None else seed, "cpu")
    n, c, m, nh, nI, cI, dt = p["n"], p["c"], p["m"], p["n_h"], p["n_hI"], p["c_I"], p["dtype"]
    d = {}
    for key in ("Ca", "Cb", "Za", "Zb"):
        d[key] = normal((n, c), g, 1.0, dt)
    d["q"] = normal((n, nh, c), g, 1.0, dt)
    d["qI"] = normal((n, nI, cI), g, 1.0, dt)
    d["KIcomp"] = normal((n // m, cI), g, 1.0, dt)
    d["w"] = softplus_normal((n, nI), g)
    d["Ba"] = normal((m, c), g, 0.1, dt)
    d["Bb"] = normal((m, c), g, 0.1, dt)
    d["sink"] = normal((nh,), g, 1.0, torch.float32)
    d["kv_raw"] = d["Ca"]
    d["scale"] = 1.0 / math.sqrt(c)
    d["params"] = p
    return d


def compress_inputs(overlap=True, n=None, c=None, m=None, dtype=None, seed=None, device="cpu", b=1):
    """Compressor sweep inputs: [b, n, c] streams and [m, c] biases."""
    p = dict(COMPRESS)
    n = p["n"] if n is None else n
    c = p["c"] if c is None else c
    dt = p["dtype"] if dtype is None else dtype
    seed = p["seed"] if seed is None else seed
    g = _gen(seed, device)
    if overlap:
        m = p["m"] if m is None else m
        d = {
            "Ca": normal((b, n, c), g, 1.0, dt, device), "Cb": normal((b, n, c), g, 1.0, dt, device),
            "Za": normal((b, n, c), g, 2.0, dt, device), "Zb": normal((b, n, c), g, 2.0, dt, device),
            "Ba": normal((m, c), g, 0.1, dt, device), "Bb": normal((m, c), g, 0.1, dt, device),
        }
    else:
        m = p["m_prime"] if m is None else m
        d = {"C": normal((b, n, c), g, 1.0, dt, device), "Z": normal((b, n, c), g, 2.0, dt, device),
             "B": normal((m, c), g, 0.1, dt, device)}
    d["m"] = m
    return d


def prefill_inputs(n=None, seed=None, device="cpu", n_h=None, k=None, unscaled=False):
    """CSA prefill layer at the Flash-like shape (optionally shortened).

    unscaled=True draws every tensor from N(0,1) instead (a sharper-softmax
    test case at the same head shapes)."""
    p = dict(PREFILL)
    if n is not None:
        p["n"] = n
    if n_h is not None:
        p["n_h"] = n_h
    if k is not None:
        p["k"] = k
    g = _gen(p["seed"] if seed is None else seed, device)
    n, c, m, nh, nI, cI, dt = p["n"], p["c"], p["m"], p["n_h"], p["n_hI"], p["c_I"], p["dtype"]
    draw = (lambda shape: normal(shape, g, 1.0, dt, device)) if unscaled else \
        (lambda shape: scaled(shape, g, dt, device))
    d = {}
    d["q"] = draw((n, nh, c))
    d["qI"] = draw((n, nI, cI))
    for key in ("Ca", "Cb", "Za", "Zb"):
        d[key] = draw((n, c))
    d["KIcomp"] = draw((n // m, cI))
    d["Ba"] = draw((m, c))
    d["Bb"] = draw((m, c))
    for key in ("ICa", "ICb", "IZa", "IZb"):
        d[key] = draw((n, cI))
    d["IBa"] = draw((m, cI))
    d["IBb"] = draw((m, cI))
    d["w"] = softplus_normal((n, nI), g, device)
    d["sink"] = normal((nh,), g, 1.0, torch.float32, device)
    d["kv_raw"] = d["Ca"]
    d["scale"] = 1.0 / math.sqrt(c)
    d["params"] = p
    return d


def norm_rope_inputs(rows, heads, c, dtype=torch.bfloat16, seed=0, device="cpu", std=3.0, gain=True):
    """Vectors x [rows, heads, c] ~ N(0, std^2) and per-dimension norm gains
    gamma [c] = 1 + N(0, 0.1^2) in float32 (None when gain is False)."""
    g = _gen(seed, device)
    x = normal((rows, heads, c), g, std, dtype, device)
    gamma = (1.0 + normal((c,), g, 0.1, torch.float32, device)) if gain else None
    return x, gamma


def out_proj_inputs(n, n_h, c, g, d_g, d, seed=0, device="cpu", dtype=torch.bfloat16):
    """Grouped output projection: head outputs o [n, n_h, c] ~ N(0,1) and
    weights WG [g, d_g, (n_h/g) c], WO [d, g d_g], each N(0,1) / sqrt(fan-in)."""
    gen = _gen(seed, device)
    o = normal((n, n_h, c), gen, 1.0, dtype, device)
    WG = scaled((g, d_g, (n_h // g) * c), gen, dtype, device)
    WO = scaled((d, g * d_g), gen, dtype, device)
    return o, WG, WO


def hca_inputs(n=None, seed=None, device="cpu", n_h=None, m_prime=None):
    """HCA prefill layer; q is the big tensor ([n, n_h, c])."""
    p = dict(HCA)
    for key, v in (("n", n), ("n_h", n_h), ("m_prime", m_prime)):
        if v is not None:
            p[key] = v
    g = _gen(p["seed"] if seed is None else seed, device)
    n, c, mp, nh, dt = p["n"], p["c"], p["m_prime"], p["n_h"], p["dtype"]
    d = {"C": scaled((n, c), g, dt, device), "Z": scaled((n, c), g, dt, device),
         "B": scaled((mp, c), g, dt, device)}
    d["q"] = scaled((n, nh, c), g, dt, device)
    d["sink"] = normal((nh,), g, 1.0, torch.float32, device)
    d["kv_raw"] = d["C"]
    d["scale"] = 1.0 / math.sqrt(c)
    d["params"] = p
    return d


def decode_inputs(seed=None, device="cpu", b=None, history=None, steps=None, cap_extra=16):
    """Long-context decode state and the per-step tokens.

    Caches are allocated with `cap_extra` spare rows so that the decode
    steps can append entries in place."""
    p = dict(DECODE)
    for key, v in (("b", b), ("history", history), ("steps", steps)):
        if v is not None:
            p[key] = v
    g = _gen(p["seed"] if seed is None else seed, device)
    b, hist, m, nh, c, nw, nI, cI, steps, dt = (p["b"], p["history"], p["m"], p["n_h"], p["c"],
                                                 p["n_win"], p["n_hI"], p["c_I"], p["steps"], p["dtype"])
    ne = hist // m
    d = {}
    Cc = torch.empty((b, ne + cap_extra, c), dtype=dt, device=device)
    Cc[:, :ne] = scaled((b, ne, c), g, dt, device)
    Cc[:, ne:] = 0
    KI = torch.empty((b, ne + cap_extra, cI), dtype=dt, device=device)
    KI[:, :ne] = scaled((b, ne, cI), g, dt, device)
    KI[:, ne:] = 0
    d["Ccomp"], d["KIcomp"], d["n_comp0"] = Cc, KI, ne
    # window buffer: n_win rows before the first step plus room for the steps
    win = torch.zeros((b, nw + steps, c), dtype=dt, device=device)
    win[:, :nw] = scaled((b, nw, c), g, dt, device)
    d["window"], d["window_pos0"] = win, hist - nw
    # previous complete block's stream-b state (main and indexer keys)
    d["prev_Cb"] = scaled((b, m, c), g, dt, device)
    d["prev_Zb"] = scaled((b, m, c), g, dt, device)
    d["prev_ICb"] = scaled((b, m, cI), g, dt, device)
    d["prev_IZb"] = scaled((b, m, cI), g, dt, device)
    for key, dim in (("Ba", c), ("Bb", c), ("IBa", cI), ("IBb", cI)):
        d[key] = scaled((m, dim), g, dt, device)
    d["sink"] = normal((nh,), g, 1.0, torch.float32, device)
    # per-step tokens: rows of the four main and four indexer-key streams
    d["tok"] = {key: scaled((steps, b, c), g, dt, device) for key in ("Ca", "Cb", "Za", "Zb")}
    d["tok"].update({key: scaled((steps, b, cI), g, dt, device) for key in ("ICa", "ICb", "IZa", "IZb")})
    d["q"] = scaled((steps, b, 1, nh, c), g, dt, device)
    d["qI"] = scaled((steps, b, 1, nI, cI), g, dt, device)
    d["w"] = softplus_normal((steps, b, 1, nI), g, device)
    d["scale"] = 1.0 / math.sqrt(c)
    d["params"] = p
    return d
