"""Plain CPU oracle for one layer of compressed sparse attention (CSA) and its
heavier-compression sibling (HCA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the test suite, the smoke check in the repository's
entry module and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP library and never reads anything the GPU produced.

Every routine is the plain definition written out in float64 NumPy, looping
or broadcasting in the order the pages state; none is blocked, fused or
reordered for speed.  Sources (web pages, cited by site, title and section):

  [P1] polysight "06-formulas" (Liang Wenfeng voices), section B9 "CSA + HCA"
  [P2] songhuiming "DeepSeek-V4 百万 token 上下文", sections 4.1-4.5, 5.1-5.2, 7
  [P3] AirCoding "deepseek-paper-analysis", sections 7.1-7.3 and 7.6
  [P5] cooking-agi "DeepSeek-V4: 压缩历史以后，还能读到什么？", sections 2-3

Readings taken where the pages are silent or garbled (each also listed in the
design notes):
  * causal visibility: a query at 0-based position t may read compressed entry
    s iff s < (t + 1) // m ([P5] section 3; [P1]/[P2] write floor(t/m), which
    would hide an entry that is already complete at t = m(i+1) - 1);
  * the compressor softmax runs over the 2m rows separately for every one of
    the c dimensions ([P2] section 4.1: the 2m weights sum to one per dim);
  * the sink logit adds exp(z'_h) to the softmax denominator only and is not
    multiplied by the softmax scale ([P1] B9, [P2] sections 4.5/7.3);
  * softmax scale is an explicit argument (1/sqrt(c) by default); the pages
    never state it;
  * index ties: the lower entry index wins the last slot; indices are returned
    ascending and padded with -1;
  * fewer than k visible entries: all of them are read ([P1] B9 read count
    min(k, n/m); [P5] section 2 ledger);
  * the sliding window for position t holds raw rows max(0, t-n_win+1)..t and
    is kept separate from the compressed entries, never de-duplicated ([P5]
    section 2);
  * the low-precision indexer ([P1] B9 estimate paragraph and B11; [P2]
    section 13.3; [P3] section 7, FP4 quantization-aware training): the
    indexer queries and keys are taken as 8-bit E4M3 codes, or as OCP MXFP4
    (E2M1 elements, one E8M0 power-of-two scale per 32 consecutive
    dimensions); the scores are the same weighted ReLU sums of the values the
    codes stand for;
  * normalisation and partial RoPE ([P2] section 4.5, [P3] section 7.1): RMSNorm
    with a per-dimension gain and explicit eps, then rotation of the last 64
    dimensions as adjacent pairs with frequencies base^(-2i/64); a compressed
    entry sits at the position of its block's first token; the attention
    output is rotated back by -t;
  * grouped output projection ([P2] section 4.4): groups of consecutive
    heads, each group's heads concatenated in head order, the group results
    concatenated in group order; weights stored with the input dimension
    contiguous ([g, d_g, (n_h/g) c] and [d, g d_g]).

parity unpinned: none of the routines here.  Each has at least one test that
pins it to something other than itself (closed forms, invariants, library
routines, brute force or the pages' worked numbers).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


# --------------------------------------------------------------------------
# Causality and the read ledger
# --------------------------------------------------------------------------

def visible_entries(t: int, m: int) -> int:
    """Number of compressed entries a query at 0-based position t may read.

    [P5] section 3 (future leakage): after the query at t has been processed
    t + 1 positions exist; an entry is complete once all m of its tokens are,
    so (t + 1) // m entries are complete.  Worked checks on that page with
    block width 4: t = 7 reads the second entry, t = 8 may not read the entry
    covering 8..11.
    """
    if t < 0 or m <= 0:
        raise ValueError("t must be >= 0 and m > 0")
    return (t + 1) // m


@dataclass(frozen=True)
class LayerReads:
    """What one query of one compressed layer stores and reads."""
    stored: int   # completed compressed entries
    tail: int     # processed tokens still waiting in the open block
    reads: int    # entries in the main attention's softmax (window included)


def layer_reads(history: int, ratio: int, n_win: int, k: int | None = None) -> LayerReads:
    """Entries a query reads in one layer, after `history` processed positions.

    Closed form of [P1] B9 (per-query read count of a CSA layer is
    min(k, n/m) + n_win, of an HCA layer n/m' + n_win) with the completed
    count of [P5] section 3 ((t + 1) // m at the newest position t =
    history - 1).  k = None is the dense HCA read of every completed entry;
    a window never holds more rows than exist.  The worked values of [P5]
    section 2 pin it.
    """
    done = visible_entries(history - 1, ratio)
    picked = done if k is None else min(int(k), done)
    return LayerReads(stored=done, tail=history - done * ratio,
                      reads=picked + min(history, int(n_win)))


# --------------------------------------------------------------------------
# Compressors
# --------------------------------------------------------------------------

def compress_weights_overlap(Za, Zb, Ba, Bb, m: int, prev_Zb=None):
    """Per-dimension softmax weights of the overlapped CSA compressor.

    [P1] B9 / [P2] section 4.1 (Eq. 11): entry i scores the m rows of block i
    from stream a (Z^a + B^a) and the m rows of block i-1 from stream b
    (Z^b + B^b); the 2m scores are normalised jointly, separately for each
    dimension.  Block -1 is padded with -inf scores ([P2] section 4.1).

    Returns (Sa, Sb), each [n//m, m, c].
    """
    Za, Zb, Ba, Bb = _f64(Za), _f64(Zb), _f64(Ba), _f64(Bb)
    n, c = Za.shape
    ne = n // m
    # scores of the current block, stream a, with the intra-block bias
    ua = Za[: ne * m].reshape(ne, m, c) + Ba[None, :, :]
    # scores of the previous block, stream b: block i-1 for entry i
    prev = np.full((1, m, c), -np.inf) if prev_Zb is None else _f64(prev_Zb).reshape(1, m, c)
    zb_blocks = Zb[: ne * m].reshape(ne, m, c)
    zb_prev = np.concatenate([prev, zb_blocks[: ne - 1]], axis=0)[:ne]
    ub = zb_prev + Bb[None, :, :]
    u = np.concatenate([ua, ub], axis=1)           # [ne, 2m, c]
    u_max = u.max(axis=1, keepdims=True)
    e = np.exp(u - u_max)
    S = e / e.sum(axis=1, keepdims=True)
    return S[:, :m, :], S[:, m:, :]


def compress_overlap(Ca, Cb, Za, Zb, Ba, Bb, m: int, prev_Cb=None, prev_Zb=None):
    """Overlapped CSA compressor, one sequence: [n, c] streams -> [n//m, c].

    [P1] B9 / [P2] section 4.1 (Eq. 12): C^Comp_i is the sum over the m rows
    of block i of S^a (.) C^a plus the sum over the m rows of block i-1 of
    S^b (.) C^b, where (.) is the element-wise product.  Block -1 has zero
    values ([P2] section 4.1).  `prev_Cb`/`prev_Zb` ([m, c]) stand for block
    -1 when the rows given here continue an earlier sequence (decode state,
    [P3] section 7.6 state cache).
    """
    if (prev_Cb is None) != (prev_Zb is None):
        raise ValueError("prev_Cb and prev_Zb come together")
    Ca, Cb = _f64(Ca), _f64(Cb)
    n, c = Ca.shape
    ne = n // m
    Sa, Sb = compress_weights_overlap(Za, Zb, Ba, Bb, m, prev_Zb)
    ca = Ca[: ne * m].reshape(ne, m, c)
    prev = np.zeros((1, m, c)) if prev_Cb is None else _f64(prev_Cb).reshape(1, m, c)
    cb = np.concatenate([prev, Cb[: ne * m].reshape(ne, m, c)[: ne - 1]], axis=0)[:ne]
    return (Sa * ca).sum(axis=1) + (Sb * cb).sum(axis=1)


def compress_weights_pool(Z, B, m_prime: int):
    """Per-dimension softmax weights of the HCA compressor, [n//m', m', c].

    [P1] B9 / [P2] section 5.1 / [P3] section 7.2: a single stream, the m'
    rows of one block, no overlap with the previous block.
    """
    Z, B = _f64(Z), _f64(B)
    n, c = Z.shape
    ne = n // m_prime
    u = Z[: ne * m_prime].reshape(ne, m_prime, c) + B[None, :, :]
    e = np.exp(u - u.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def compress_pool(C, Z, B, m_prime: int):
    """HCA compressor, one sequence: [n, c] -> [n//m', c] (same sources)."""
    C = _f64(C)
    n, c = C.shape
    ne = n // m_prime
    S = compress_weights_pool(Z, B, m_prime)
    return (S * C[: ne * m_prime].reshape(ne, m_prime, c)).sum(axis=1)


# --------------------------------------------------------------------------
# Lightning indexer and top-k
# --------------------------------------------------------------------------

def index_scores(qI, w, KI, t_pos, m: int, chunk: int = 64):
    """Indexer scores I[t, s] for queries at positions t_pos.

    [P1] B9 / [P3] section 7.1: I_{t,s} = sum over indexer heads h of
    w_{t,h} * ReLU(q^I_{t,h} . K^IComp_s).  Entries a query may not read
    (s >= (t+1)//m) get -inf.

    qI [n_q, n_hI, c_I], w [n_q, n_hI], KI [n_comp, c_I] -> [n_q, n_comp].
    Queries are processed `chunk` at a time only to bound memory.
    """
    qI, w, KI = _f64(qI), _f64(w), _f64(KI)
    n_q = qI.shape[0]
    n_comp = KI.shape[0]
    t_pos = np.asarray(t_pos, dtype=np.int64)
    out = np.full((n_q, n_comp), -np.inf)
    for a in range(0, n_q, chunk):
        b = min(n_q, a + chunk)
        dots = qI[a:b] @ KI.T                      # [T, n_hI, n_comp]
        sc = (w[a:b, :, None] * np.maximum(dots, 0.0)).sum(axis=1)
        for r in range(a, b):
            v = min(visible_entries(int(t_pos[r]), m), n_comp)
            out[r, :v] = sc[r - a, :v]
    return out


def fp8_e4m3_decode(codes):
    """Values of 8-bit E4M3 codes (uint8 array), float64.

    The low-precision indexer of [P1] B9 (estimate paragraph) and B11 runs
    the indexer's query/key path in a narrow float format; the format taken
    here is 8-bit E4M3 of the OCP 8-bit floating point specification:
    bit 7 sign, bits 6-3 exponent e (bias 7), bits 2-0 mantissa f; e = 0
    gives the subnormals (f / 8) * 2^-6, e > 0 gives (1 + f / 8) * 2^(e - 7);
    there are no infinities, and the two codes with e = 15, f = 7 are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 3) & 15
    f = (c & 7).astype(F64)
    mag = np.where(e == 0, (f / 8.0) * 2.0 ** -6, (1.0 + f / 8.0) * np.exp2((e - 7).astype(F64)))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


def fp8_e4m3_encode(x):
    """E4M3 codes of finite values |x| <= 448: the nearest representable
    value, ties to the code with an even mantissa (round to nearest even),
    the sign kept for negative values (a negative value that rounds to 0
    keeps its sign bit).  Brute force over the 127 non-negative finite codes
    decoded by fp8_e4m3_decode, so the two share the format's definition."""
    x = _f64(x)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > 448.0):
        raise ValueError("E4M3 holds finite values up to 448")
    grid = fp8_e4m3_decode(np.arange(127, dtype=np.uint8))          # codes 0x00..0x7E, increasing
    a = np.abs(x).reshape(-1)
    out = np.empty(a.shape, dtype=np.uint8)
    for lo in range(0, a.size, 1 << 16):
        blk = a[lo:lo + (1 << 16)]
        d = np.abs(blk[:, None] - grid[None, :])
        best = d.min(axis=1, keepdims=True)
        tie = d == best
        # among the nearest codes (at most two), the even one
        even = tie & (np.arange(127)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
        out[lo:lo + blk.size] = pick
    out = out.reshape(x.shape)
    return np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)


def kv_fp8_encode(E, rope_dims: int = 64):
    """Mixed-precision storage of KV entries ([P3] section 7.3, KV mixed
    precision storage; [P1] B9: the RoPE dimensions stay BF16, the other
    dimensions are FP8).  Readings: the RoPE dimensions are the last
    rope_dims (the partial RoPE of [P2] section 4.5 rotates the last 64);
    the FP8 format is E4M3 with one power-of-two scale per entry, the
    smallest 2^e with max |x| / 2^e <= 448 (2^0 for an all-zero entry), so
    that every entry uses the format's whole range.  E [n, c] holds the
    values to store (the RoPE part is kept as given).
    Returns (codes [n, c - rope_dims] uint8, rope [n, rope_dims] float64,
    scale [n] float64)."""
    E = _f64(E)
    head = E[:, : E.shape[1] - rope_dims]
    amax = np.abs(head).max(axis=1) if head.shape[1] else np.zeros(E.shape[0])
    e = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0.0)
    scale = np.exp2(e)
    # max |x| / scale may exceed 448 by rounding of log2: step up once more
    over = np.abs(head).max(axis=1, initial=0.0) / scale > 448.0
    scale = np.where(over, scale * 2.0, scale)
    codes = fp8_e4m3_encode(head / scale[:, None])
    return codes, E[:, E.shape[1] - rope_dims:].copy(), scale


def kv_fp8_decode(codes, rope, scale):
    """Values of entries stored by kv_fp8_encode: decoded E4M3 codes times
    the entry's scale, then the RoPE dimensions."""
    return np.concatenate([fp8_e4m3_decode(codes) * _f64(scale)[:, None], _f64(rope)], axis=1)


def e2m1_decode(nibbles):
    """Values of 4-bit E2M1 codes (integer array of 0..15), float64.

    OCP Microscaling Formats (MX) specification v1.0, FP4 element: bit 3
    sign, bits 2-1 exponent e (bias 1), bit 0 mantissa f; e = 0 gives the
    subnormals f / 2, e > 0 gives (1 + f / 2) * 2^(e - 1).  No infinities or
    NaN.  [P2] section 13.3 and [P3] section 7 put the indexer's query/key
    path in this 4-bit format.
    """
    c = np.asarray(nibbles).astype(np.int64) & 15
    sign = np.where(c >= 8, -1.0, 1.0)
    e = (c >> 1) & 3
    f = (c & 1).astype(F64)
    mag = np.where(e == 0, f / 2.0, (1.0 + f / 2.0) * np.exp2((e - 1).astype(F64)))
    return sign * mag


def e8m0_decode(codes):
    """Values of 8-bit E8M0 scales (uint8 array), float64: 2^(s - 127), and
    NaN for s = 255 (OCP MX specification v1.0, shared scale)."""
    s = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2((s - 127).astype(F64)))


def mxfp4_decode(codes, scales, block: int = 32):
    """Values of MXFP4 vectors, float64 [..., c].

    codes [..., c / 2] uint8: byte j holds element 2j in its low nibble and
    element 2j + 1 in its high nibble; scales [..., c / block] uint8 E8M0:
    element d is e2m1(code of d) * e8m0(scale of block d // block) (OCP MX
    specification v1.0: one shared scale per block of 32 elements).
    """
    b = np.asarray(codes, dtype=np.uint8)
    lo = e2m1_decode(b & 15)
    hi = e2m1_decode(b >> 4)
    el = np.stack([lo, hi], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])
    sc = np.repeat(e8m0_decode(scales), block, axis=-1)
    return el * sc


def mxfp4_encode(x, block: int = 32):
    """OCP MXFP4 encoding of x [..., c] (c a multiple of 32), float64 steps.

    OCP MX specification v1.0, conversion to an MX format: each block of 32
    takes the shared scale X = 2^(floor(log2 max|x|) - 2) (2 is the largest
    E2M1 exponent), every element x / X is rounded to the nearest E2M1
    magnitude, ties to the even code, and saturated at 6.  Reading taken
    where the specification leaves a choice: an all-zero block gets scale
    byte 0 (2^-127); the sign bit is set for x < 0 also when the magnitude
    rounds to 0.  Returns (codes [..., c/2] uint8, element 2j in the low
    nibble of byte j; scales [..., c/32] uint8, E8M0 biased by 127).
    """
    v = _f64(x)
    *lead, c = v.shape
    blk = v.reshape(*lead, c // block, block)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))          # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127).clip(-127, 127)   # floor(log2 amax) - 2
    y = np.abs(blk) / np.exp2(e.astype(F64))[..., None]
    # nearest of 0, .5, 1, 1.5, 2, 3, 4, 6; on a midpoint the even code
    # (mantissa bit 0) wins: the midpoints after codes 1, 3, 5 round up
    mids = [(0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False)]
    code = np.zeros(y.shape, dtype=np.int64)
    for mid, up in mids:
        code += (y >= mid) if up else (y > mid)
    code = code + np.where(blk < 0, 8, 0)
    code = code.reshape(*lead, c)
    codes = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def topk_select(scores_row, v: int, k: int):
    """Indices of the top-k among the first v scores of one query.

    [P1] B9 / [P3] section 7.1: the entries whose scores are among the k
    largest of I_{t,:}; all v if v <= k.  Reading: the lower index wins a tie;
    the result is ascending and padded with -1 to length k.
    """
    s = np.arange(v)
    order = np.lexsort((s, -_f64(scores_row)[:v]))   # by score desc, then s asc
    take = np.sort(order[: min(k, v)])
    out = np.full(k, -1, dtype=np.int64)
    out[: take.size] = take
    return out


def index_topk(qI, w, KI, t_pos, m: int, k: int):
    """Indexer scores followed by top-k, per query: (idx [n_q,k], scores)."""
    sc = index_scores(qI, w, KI, t_pos, m)
    n_comp = KI.shape[0]
    idx = np.stack([
        topk_select(sc[r], min(visible_entries(int(t), m), n_comp), k)
        for r, t in enumerate(np.asarray(t_pos))
    ]) if len(t_pos) else np.zeros((0, k), dtype=np.int64)
    return idx, sc


# --------------------------------------------------------------------------
# Core attention with window and sink
# --------------------------------------------------------------------------

def attend_entries(q_t, E, sink, scale: float):
    """Shared key/value attention of one query over an entry set, with sink.

    [P3] section 7.1 / [P2] section 4.3: each entry is both key and value and
    all n_h query heads read the same entries.  [P2] sections 4.5 and 7.3,
    [P1] B9: the compressed and the window entries share one softmax, whose
    denominator also holds exp(z'_h) of the head's sink logit; the sink adds
    no value.

    q_t [n_h, c], E [N, c], sink [n_h] -> [n_h, c].
    """
    q_t, E, sink = _f64(q_t), _f64(E), _f64(sink)
    logits = scale * (q_t @ E.T)                     # [n_h, N]
    if logits.shape[1]:
        M = np.maximum(logits.max(axis=1), sink)
    else:
        M = sink.copy()
    p = np.exp(logits - M[:, None])
    den = p.sum(axis=1) + np.exp(sink - M)
    return (p @ E) / den[:, None]


def window_rows(t: int, n_win: int):
    """Raw positions in the causal window of a query at t ([P2] section 4.5)."""
    return np.arange(max(0, t - n_win + 1), t + 1)


def csa_attend(q, Ccomp, idx, kv_raw, raw_pos0: int, sink, t_pos, n_win: int,
               scale: float, m: int | None = None):
    """CSA main attention for queries at t_pos, one sequence.

    q [n_q, n_h, c]; Ccomp [n_comp, c]; idx [n_q, k] (-1 padded); kv_raw
    [n_raw, c], row j at position raw_pos0 + j; sink [n_h].
    The entry set of query t is the selected compressed rows plus the window
    rows ([P2] section 4.5).  If m is given, selected indices must be visible.
    """
    q, Ccomp, kv_raw = _f64(q), _f64(Ccomp), _f64(kv_raw)
    out = np.zeros(q.shape, dtype=F64)
    for r, t in enumerate(np.asarray(t_pos)):
        t = int(t)
        sel = np.asarray(idx[r])
        sel = sel[sel >= 0]
        if m is not None and sel.size:
            assert sel.max() < visible_entries(t, m), "index reads the future"
        win = window_rows(t, n_win) - raw_pos0
        assert win.min() >= 0 and win.max() < kv_raw.shape[0], "window outside kv_raw"
        E = np.concatenate([Ccomp[sel], kv_raw[win]], axis=0)
        out[r] = attend_entries(q[r], E, sink, scale)
    return out


def hca_attend(q, Ccomp, kv_raw, raw_pos0: int, sink, t_pos, m_prime: int,
               n_win: int, scale: float):
    """HCA dense attention: every completed compressed entry plus the window.

    [P1] B9 / [P2] section 5.2 / [P3] section 7.2: no indexer, no selection;
    the entry set of query t is C^Comp_s for s < (t+1)//m' plus the window.
    """
    q, Ccomp, kv_raw = _f64(q), _f64(Ccomp), _f64(kv_raw)
    out = np.zeros(q.shape, dtype=F64)
    for r, t in enumerate(np.asarray(t_pos)):
        t = int(t)
        v = min(visible_entries(t, m_prime), Ccomp.shape[0])
        win = window_rows(t, n_win) - raw_pos0
        E = np.concatenate([Ccomp[:v], kv_raw[win]], axis=0)
        out[r] = attend_entries(q[r], E, sink, scale)
    return out


def hca_layer(C, Z, B, q, kv_raw, sink, m_prime: int, n_win: int, scale: float,
              t_rows=None):
    """Whole HCA prefill of one sequence: compress, then dense attention.

    `t_rows` optionally restricts the queries evaluated (all by default).
    Returns (Ccomp, out[t_rows]).
    """
    Ccomp = compress_pool(C, Z, B, m_prime)
    n = _f64(C).shape[0]
    rows = np.arange(n) if t_rows is None else np.asarray(t_rows)
    out = hca_attend(_f64(q)[rows], Ccomp, kv_raw, 0, sink, rows, m_prime, n_win, scale)
    return Ccomp, out


def csa_layer(streams, istreams, q, qI, w, kv_raw, sink, m: int, k: int,
              n_win: int, scale: float, t_rows=None):
    """Whole CSA prefill of one sequence.

    streams = (Ca, Cb, Za, Zb, Ba, Bb) for the main entries; istreams the same
    six arrays for the indexer keys, "compressed the same way" ([P2] section
    4.2, step 1).  Returns (Ccomp, KIcomp, idx, out) for the query rows.
    """
    Ccomp = compress_overlap(*streams, m)
    KIcomp = compress_overlap(*istreams, m)
    n = _f64(q).shape[0]
    rows = np.arange(n) if t_rows is None else np.asarray(t_rows)
    idx, _ = index_topk(_f64(qI)[rows], _f64(w)[rows], KIcomp, rows, m, k)
    out = csa_attend(_f64(q)[rows], Ccomp, idx, kv_raw, 0, sink, rows, n_win, scale, m)
    return Ccomp, KIcomp, idx, out


# --------------------------------------------------------------------------
# Normalisation and partial rotary embedding around the core attention
# ([P2] section 4.5 "other details"; [P3] section 7.1 "Partial RoPE")
# --------------------------------------------------------------------------

def rms_norm(x, gamma, eps: float):
    """RMSNorm along the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    [P2] section 4.5: every query head and every KV entry is normalised this
    way before the core attention, which keeps the logits bounded.  Readings:
    one learned gain per dimension (gamma [c]) and an explicit eps; the pages
    give neither.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gamma)


def rope_frequencies(dims: int, base: float):
    """Angular frequency of rotation pair i < dims/2: base^(-2i/dims).

    Reading: the standard rotary frequencies; [P2] section 4.5 and [P3]
    section 7.1 name RoPE on the last 64 dimensions without its constants.
    """
    i = np.arange(dims // 2, dtype=F64)
    return float(base) ** (-2.0 * i / dims)


def rope(x, pos, dims: int, base: float):
    """Rotary embedding of the last `dims` dimensions at the given positions.

    x [rows, ..., c], pos [rows] (any integers, negative included).  Pair i is
    the adjacent dimensions (c - dims + 2i, c - dims + 2i + 1), read as the
    complex number a + ib and multiplied by exp(i * pos * theta_i) (reading:
    interleaved pairs; the pages do not say how the 64 dimensions pair up).
    The other c - dims dimensions are unchanged.
    """
    x = _f64(x).copy()
    c = x.shape[-1]
    lo = c - dims
    ang = np.asarray(pos, dtype=F64).reshape((-1,) + (1,) * (x.ndim - 1)) * rope_frequencies(dims, base)
    cos, sin = np.cos(ang), np.sin(ang)
    a = x[..., lo::2].copy()
    b = x[..., lo + 1::2].copy()
    x[..., lo::2] = a * cos - b * sin
    x[..., lo + 1::2] = a * sin + b * cos
    return x


def norm_rope(x, gamma, eps: float, pos, dims: int, base: float):
    """RMSNorm (skipped when gamma is None), then the rotary embedding.

    Reading: the norm comes first and its gain applies before the rotation.
    """
    y = _f64(x) if gamma is None else rms_norm(x, gamma, eps)
    return rope(y, pos, dims, base) if dims else y


def csa_attend_rope(q, Ccomp, idx, kv_raw, raw_pos0: int, sink, t_pos, n_win: int,
                    scale: float, m: int, gamma_q, gamma_kv, eps: float, dims: int,
                    base: float, entry_pos0: int = 0):
    """CSA attention with the normalisation and partial RoPE of [P2] section
    4.5 and [P3] section 7.1 around it.

    Query heads at t and KV entries are normalised and rotated at their own
    positions; the attention output's last `dims` dimensions are then rotated
    by -t, so that only relative positions remain in it.  Readings: compressed
    entry s sits at position entry_pos0 + m*s (the first token of its block),
    a raw window row at its token position; the window rows take the same
    norm gain as the compressed entries.  With m = m' and every visible entry
    selected this is the HCA form.
    """
    t_pos = np.asarray(t_pos)
    qn = norm_rope(q, gamma_q, eps, t_pos, dims, base)
    Cn = norm_rope(Ccomp, gamma_kv, eps, entry_pos0 + m * np.arange(_f64(Ccomp).shape[0]), dims, base)
    Rn = norm_rope(kv_raw, gamma_kv, eps, raw_pos0 + np.arange(_f64(kv_raw).shape[0]), dims, base)
    o = csa_attend(qn, Cn, idx, Rn, raw_pos0, sink, t_pos, n_win, scale, m)
    return rope(o, -t_pos, dims, base)


# --------------------------------------------------------------------------
# Grouped output projection ([P2] section 4.4; [P3] section 7.1)
# --------------------------------------------------------------------------

def grouped_out_proj(o, WG, WO, g: int, mid_round=None):
    """u_t = W^O [W^G_1 o^1_t; ...; W^G_g o^g_t].

    [P2] section 4.4: the n_h head outputs of a token are split into g groups
    of n_h/g consecutive heads; group j's concatenated output o^j_t (head
    order, then dimension) is projected to d_g values, and the g results,
    concatenated in group order, are projected to d.  [P3] section 7.1 gives
    the Flash shape g = 8, d_g = 1024, d = 4096.
    o [n, n_h, c]; WG [g, d_g, (n_h/g)*c] (group j maps o^j to W^G_j o^j);
    WO [d, g*d_g].  Returns (mid [n, g*d_g], u [n, d]).  mid_round, when
    given, is applied to mid before the second projection (the storage format
    of an intermediate kept between two calls).
    """
    o, WG, WO = _f64(o), _f64(WG), _f64(WO)
    n, n_h, c = o.shape
    hpg = n_h // g
    parts = [o[:, j * hpg:(j + 1) * hpg, :].reshape(n, hpg * c) @ WG[j].T for j in range(g)]
    mid = np.concatenate(parts, axis=1)
    mid2 = mid if mid_round is None else _f64(mid_round(mid))
    return mid, mid2 @ WO.T


# --------------------------------------------------------------------------
# Decode state ([P3] section 7.6 state cache; [P5] section 2 tails)
# --------------------------------------------------------------------------

@dataclass
class CsaDecodeState:
    """Per-sequence CSA decode state.

    [P3] section 7.6: a fixed-size state cache holds the n_win most recent
    uncompressed entries and the tokens still waiting to be compressed; [P5]
    section 2 adds that CSA must also keep the previous block's overlap state.
    Compressed entries (main and indexer keys) accumulate in growing caches.
    """
    m: int
    n_win: int
    c: int
    c_I: int
    Ccomp: list = field(default_factory=list)
    KIcomp: list = field(default_factory=list)
    window: list = field(default_factory=list)          # (position, row)
    tail: list = field(default_factory=list)            # rows of the open block
    prev_b: tuple | None = None                         # (Cb, Zb, ICb, IZb) of last full block
    t: int = -1

    def append(self, row: dict, biases: dict):
        """Add token t+1; emit one entry of each cache when its block fills."""
        self.t += 1
        self.window.append((self.t, _f64(row["Ca"])))
        self.window = self.window[-self.n_win:]
        self.tail.append({k: _f64(v) for k, v in row.items()})
        if len(self.tail) == self.m:
            blk = {k: np.stack([r[k] for r in self.tail]) for k in self.tail[0]}
            pc, pz, pic, piz = self.prev_b if self.prev_b else (None, None, None, None)
            e = compress_overlap(blk["Ca"], blk["Cb"], blk["Za"], blk["Zb"],
                                 biases["Ba"], biases["Bb"], self.m, pc, pz)
            ei = compress_overlap(blk["ICa"], blk["ICb"], blk["IZa"], blk["IZb"],
                                  biases["IBa"], biases["IBb"], self.m, pic, piz)
            self.Ccomp.append(e[0])
            self.KIcomp.append(ei[0])
            self.prev_b = (blk["Cb"], blk["Zb"], blk["ICb"], blk["IZb"])
            self.tail = []

    def query(self, q_t, qI_t, w_t, sink, k: int, scale: float):
        """Index, select and attend for the newest token's query."""
        t = self.t
        KI = np.array(self.KIcomp).reshape(-1, self.c_I)
        Cc = np.array(self.Ccomp).reshape(-1, self.c)
        idx, _ = index_topk(_f64(qI_t)[None], _f64(w_t)[None], KI, [t], self.m, k)
        pos0 = self.window[0][0]
        raw = np.stack([r for _, r in self.window])
        out = csa_attend(_f64(q_t)[None], Cc, idx, raw, pos0, sink, [t], self.n_win, scale, self.m)
        return idx[0], out[0]


# --------------------------------------------------------------------------
# Backward pass ([P3] section 7.6: training needs gradients of the layer;
# the pages ask that the backward reductions be deterministic)
# --------------------------------------------------------------------------

def attend_entries_backward(q_t, E, sink, scale: float, g_t):
    """Gradients of o = attend_entries(q_t, E, sink, scale) given dL/do = g_t.

    Differentiating the softmax with the sink (weights p_j over the entries,
    p_z for the sink, o = sum_j p_j e_j):
      dl_j = p_j (g . e_j - g . o)         (logit l_j = scale q . e_j)
      dz   = -p_z (g . o)                  (sink logit)
      dq   = scale sum_j dl_j e_j
      de_j = p_j g + scale dl_j q          (each entry is key and value)
    per head, the entries shared by all heads (their gradients summed).
    q_t, g_t [n_h, c]; E [N, c]; returns (dq [n_h, c], dE [N, c], dz [n_h]).
    """
    q_t, E, sink, g_t = _f64(q_t), _f64(E), _f64(sink), _f64(g_t)
    logits = scale * (q_t @ E.T)                             # [n_h, N]
    mx = np.maximum(logits.max(axis=1, initial=-np.inf), sink)
    w = np.exp(logits - mx[:, None])
    wz = np.exp(sink - mx)
    den = w.sum(axis=1) + wz
    p = w / den[:, None]
    pz = wz / den
    o = p @ E                                                # [n_h, c]
    go = (g_t * o).sum(axis=1)                               # g . o per head
    ge = g_t @ E.T                                           # g . e_j
    dl = p * (ge - go[:, None])
    dq = scale * (dl @ E)
    dE = p.T @ g_t + scale * (dl.T @ q_t)
    dz = -pz * go
    return dq, dE, dz


def csa_attend_backward(q, Ccomp, idx, kv_raw, raw_pos0: int, sink, t_pos, n_win: int,
                        scale: float, dout, m: int | None = None):
    """Gradients of csa_attend with respect to q, Ccomp, kv_raw and sink.

    The entry set of each query is the forward's (selected rows, then the
    window); an entry's gradient is the sum over every query and head that
    read it.  Returns (dq [n_q, n_h, c], dCcomp like Ccomp, dkv_raw like
    kv_raw, dsink [n_h]).
    """
    q, Ccomp, kv_raw, dout = _f64(q), _f64(Ccomp), _f64(kv_raw), _f64(dout)
    dq = np.zeros_like(q)
    dC = np.zeros_like(Ccomp)
    dR = np.zeros_like(kv_raw)
    dsink = np.zeros(q.shape[1])
    for r, t in enumerate(np.asarray(t_pos)):
        t = int(t)
        sel = np.asarray(idx[r])
        sel = sel[sel >= 0]
        if m is not None and sel.size:
            assert sel.max() < visible_entries(t, m), "index reads the future"
        win = window_rows(t, n_win) - raw_pos0
        E = np.concatenate([Ccomp[sel], kv_raw[win]], axis=0)
        dq[r], dE, dz = attend_entries_backward(q[r], E, sink, scale, dout[r])
        np.add.at(dC, sel, dE[: sel.size])
        dR[win] += dE[sel.size:]
        dsink += dz
    return dq, dC, dR, dsink


def hca_attend_backward(q, Ccomp, kv_raw, raw_pos0: int, sink, t_pos, m_prime: int,
                        n_win: int, scale: float, dout):
    """Gradients of hca_attend (every completed entry plus the window)."""
    Ccomp = _f64(Ccomp)
    n_comp = Ccomp.shape[0]
    idx = np.stack([np.concatenate([np.arange(min(visible_entries(int(t), m_prime), n_comp)),
                                    np.full(n_comp, -1)])[:max(n_comp, 1)]
                    for t in np.asarray(t_pos)]) if len(t_pos) else np.zeros((0, 1), dtype=np.int64)
    return csa_attend_backward(q, Ccomp, idx, kv_raw, raw_pos0, sink, t_pos, n_win, scale, dout, m_prime)


def compress_overlap_backward(Ca, Cb, Za, Zb, Ba, Bb, m: int, dCc, prev_Cb=None, prev_Zb=None):
    """Gradients of compress_overlap given dL/dC^Comp.

    Entry i is sum_j S_j C_j over the 2m rows (block i of stream a, block
    i-1 of stream b), S the per-dimension softmax of Z + B:
      dC_j = S_j dCc_i,   dZ_j = S_j (C_j - Cc_i) dCc_i,
    and a bias row collects dZ of that in-block row over every entry.
    Rows no entry reads (the last block's stream-b rows, a ragged tail) get
    zero.  Returns dict dCa, dCb, dZa, dZb, dBa, dBb (and dprev_Cb,
    dprev_Zb when the previous-block state is given).
    """
    Ca, Cb = _f64(Ca), _f64(Cb)
    dCc = _f64(dCc)
    n, c = Ca.shape
    ne = n // m
    Sa, Sb = compress_weights_overlap(Za, Zb, Ba, Bb, m, prev_Zb)   # [ne, m, c] each
    Cc = compress_overlap(Ca, Cb, Za, Zb, Ba, Bb, m, prev_Cb, prev_Zb)
    ca = Ca[: ne * m].reshape(ne, m, c)
    prev = np.zeros((1, m, c)) if prev_Cb is None else _f64(prev_Cb).reshape(1, m, c)
    cb = np.concatenate([prev, Cb[: ne * m].reshape(ne, m, c)[: ne - 1]], axis=0)[:ne]
    g = dCc[:, None, :]
    dca = Sa * g
    dza = Sa * (ca - Cc[:, None, :]) * g
    dcb = Sb * g
    dzb = Sb * (cb - Cc[:, None, :]) * g
    out = {k: np.zeros((n, c)) for k in ("dCa", "dCb", "dZa", "dZb")}
    out["dCa"][: ne * m] = dca.reshape(ne * m, c)
    out["dZa"][: ne * m] = dza.reshape(ne * m, c)
    # stream-b rows of block i feed entry i + 1
    if ne > 1:
        out["dCb"][: (ne - 1) * m] = dcb[1:].reshape((ne - 1) * m, c)
        out["dZb"][: (ne - 1) * m] = dzb[1:].reshape((ne - 1) * m, c)
    out["dBa"] = dza.sum(axis=0)
    out["dBb"] = dzb.sum(axis=0)
    if prev_Cb is not None and ne > 0:
        out["dprev_Cb"] = dcb[0]
        out["dprev_Zb"] = dzb[0]
    return out


def compress_pool_backward(C, Z, B, m_prime: int, dCc):
    """Gradients of compress_pool: dC, dZ [n, c] and dB [m', c]."""
    C, dCc = _f64(C), _f64(dCc)
    n, c = C.shape
    ne = n // m_prime
    S = compress_weights_pool(Z, B, m_prime)                  # [ne, m', c]
    Cc = compress_pool(C, Z, B, m_prime)
    cb = C[: ne * m_prime].reshape(ne, m_prime, c)
    g = dCc[:, None, :]
    dC = np.zeros((n, c))
    dZ = np.zeros((n, c))
    dC[: ne * m_prime] = (S * g).reshape(-1, c)
    dz = S * (cb - Cc[:, None, :]) * g
    dZ[: ne * m_prime] = dz.reshape(-1, c)
    return {"dC": dC, "dZ": dZ, "dB": dz.sum(axis=0)}


# --------------------------------------------------------------------------
# Heterogeneous decode cache ([P3] section 7.6, "Inference KV Cache")
# --------------------------------------------------------------------------

def block_geometry(m: int, m_prime: int) -> tuple:
    """Tokens per classical-cache block and the entries one block holds.

    [P3] section 7.6: a block covers lcm(m, m') raw tokens, so it holds
    lcm/m CSA entries and lcm/m' HCA entries (128, 32 and 1 for m = 4,
    m' = 128).  Returns (tokens, csa_entries, hca_entries).
    """
    if m <= 0 or m_prime <= 0:
        raise ValueError("ratios must be positive")
    tokens = m * m_prime // math.gcd(m, m_prime)
    return tokens, tokens // m, tokens // m_prime


@dataclass
class HcaDecodeState:
    """Per-request decode state of one HCA layer: a sliding window of the
    n_win most recent raw rows, the rows of the open m'-token block waiting
    for compression, and the completed entries ([P3] section 7.6; [P1] B9
    for the pooling compressor).  Window rows are the layer's C rows (the
    reading used for the HCA prefill as well)."""
    m_prime: int
    n_win: int
    entries: list = field(default_factory=list)
    window: list = field(default_factory=list)          # (position, row)
    tail: list = field(default_factory=list)            # (C, Z) rows of the open block
    t: int = -1

    def append(self, C_row, Z_row, B):
        self.t += 1
        self.window.append((self.t, _f64(C_row)))
        self.window = self.window[-self.n_win:]
        self.tail.append((_f64(C_row), _f64(Z_row)))
        if len(self.tail) == self.m_prime:
            C = np.stack([r[0] for r in self.tail])
            Z = np.stack([r[1] for r in self.tail])
            self.entries.append(compress_pool(C, Z, B, self.m_prime)[0])
            self.tail = []

    def query(self, q_t, sink, scale: float):
        """Dense attention of the newest token's query over every completed
        entry and the window."""
        t = self.t
        E = np.array(self.entries).reshape(-1, _f64(q_t).shape[-1])
        pos0 = self.window[0][0]
        raw = np.stack([r for _, r in self.window])
        return hca_attend(_f64(q_t)[None], E, raw, pos0, sink, [t], self.m_prime, self.n_win, scale)[0]

    def state_rows(self) -> int:
        """Raw rows the state holds (window + open block): bounded by
        n_win + 2 (m' - 1), whatever the request's length."""
        return len(self.window) + 2 * len(self.tail)


def default_scale(c: int) -> float:
    """Softmax scale 1/sqrt(c) (a reading: the pages never state it)."""
    return 1.0 / math.sqrt(c)
