"""Host-only checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments before any launch.

No call here reaches a kernel: every argument set is invalid (or a pure
size query), so these run without a GPU.
"""

import ctypes
import os
import re

import pytest

import long_context_compressed_csa_amd as L
from long_context_compressed_csa_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

EINVAL, ENOTSUP, ENOSPC = -1, -2, -3
FAKE = 0x10000  # a non-NULL address that is never dereferenced


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", src, flags=re.M)) - {"if"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libcsa.so is not built (run `python -m long_context_compressed_csa_amd.build`)")
    return L.load_library()


def test_header_declares_the_four_stages():
    names = _declared()
    for fn in ("csa_compress", "csa_index_topk", "csa_attend", "hca_layer"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    # and the binding declares a signature for each
    assert set(names) == set(B.SIGNATURES)


def test_version_and_strerror(lib):
    assert L.version().startswith("csa-mi355x")
    assert L.strerror(0) == "ok"
    assert "workspace" in L.strerror(ENOSPC)
    assert L.strerror(12345) == "unknown error"


def _compress(lib, **kw):
    a = dict(Ca=FAKE, Cb=FAKE, Za=FAKE, Zb=FAKE, Ba=FAKE, Bb=FAKE, pCb=None, pZb=None,
             b=1, n=16, c=8, m=4, overlap=1, dtype=1, out=FAKE, obs=0)
    a.update(kw)
    return lib.csa_compress(a["Ca"], a["Cb"], a["Za"], a["Zb"], a["Ba"], a["Bb"], a["pCb"], a["pZb"],
                            a["b"], a["n"], a["c"], a["m"], a["overlap"], a["dtype"], a["out"],
                            a["obs"], None)


def test_compress_rejects_bad_arguments(lib):
    assert _compress(lib, dtype=7) == ENOTSUP
    assert _compress(lib, m=0) == EINVAL
    assert _compress(lib, n=0) == EINVAL
    assert _compress(lib, c=-1) == EINVAL
    assert _compress(lib, Ca=None) == EINVAL
    assert _compress(lib, Cb=None) == EINVAL                 # overlap needs stream b
    assert _compress(lib, overlap=0) == EINVAL               # pooling forbids stream b
    assert _compress(lib, overlap=0, Cb=None, Zb=None, Bb=None, pCb=FAKE) == EINVAL
    assert _compress(lib, pCb=FAKE) == EINVAL                # prev state comes in pairs
    assert _compress(lib, overlap=2) == EINVAL
    assert _compress(lib, obs=5) == EINVAL                   # stride below (n/m)*c


def _topk(lib, ws_bytes=1 << 20, **kw):
    a = dict(qI=FAKE, w=FAKE, KI=FAKE, cbs=0, b=1, n_q=8, t0=0, n_comp=2, nh=2, cI=16, m=4, k=4,
             dtype=0, idx=FAKE, score=None, ws=0x100000)
    a.update(kw)
    return lib.csa_index_topk(a["qI"], a["w"], a["KI"], a["cbs"], a["b"], a["n_q"], a["t0"],
                              a["n_comp"], a["nh"], a["cI"], a["m"], a["k"], a["dtype"], a["idx"],
                              a["score"], a["ws"], ws_bytes, None)


def test_index_topk_rejects_bad_arguments(lib):
    assert _topk(lib, k=0) == EINVAL
    assert _topk(lib, m=0) == EINVAL
    assert _topk(lib, t0=-1) == EINVAL
    assert _topk(lib, n_comp=3) == EINVAL        # 8 queries from t0=0 complete only 2 entries
    assert _topk(lib, ws=None) == EINVAL
    assert _topk(lib, ws=0x100010) == EINVAL     # workspace must be 256-byte aligned
    assert _topk(lib, ws_bytes=16) == ENOSPC
    assert _topk(lib, dtype=9) == ENOTSUP
    assert _topk(lib, cbs=5) == EINVAL
    # long lists need k <= 2048 so every selection stage shrinks them
    assert _topk(lib, n_q=1, t0=4 * 10000, n_comp=10000, k=4000, ws_bytes=1 << 30) == ENOTSUP


def _topk_mx(lib, ws_bytes=1 << 20, **kw):
    a = dict(qI=FAKE, qS=FAKE, w=FAKE, KI=FAKE, KS=FAKE, cbs=0, b=1, n_q=8, t0=0, n_comp=2, nh=2, cI=64, m=4,
             k=4, idx=FAKE, score=None, ws=0x100000)
    a.update(kw)
    return lib.csa_index_topk_mxfp4(a["qI"], a["qS"], a["w"], a["KI"], a["KS"], a["cbs"], a["b"], a["n_q"],
                                    a["t0"], a["n_comp"], a["nh"], a["cI"], a["m"], a["k"], a["idx"],
                                    a["score"], a["ws"], ws_bytes, None)


def test_index_topk_mxfp4_rejects_bad_arguments(lib):
    assert _topk_mx(lib, qS=None) == EINVAL
    assert _topk_mx(lib, KS=None) == EINVAL
    assert _topk_mx(lib, cI=48) == EINVAL          # MX blocks are 32 elements
    assert _topk_mx(lib, k=0) == EINVAL
    assert _topk_mx(lib, n_comp=3) == EINVAL       # 8 queries from t0=0 complete only 2 entries
    assert _topk_mx(lib, cbs=1) == EINVAL          # fewer rows per sequence than n_comp
    assert _topk_mx(lib, ws=0x100010) == EINVAL
    assert _topk_mx(lib, ws_bytes=16) == ENOSPC
    # generic scoring holds the row's query values in LDS: n_hI * c_I <= 8192
    assert _topk_mx(lib, nh=128, cI=96) == ENOTSUP


def _quant(lib, **kw):
    a = dict(x=0x100000, xrs=64, rows=4, c=64, dtype=1, codes=0x200000, crs=32, scales=FAKE, srs=2)
    a.update(kw)
    return lib.csa_quantize_mxfp4(a["x"], a["xrs"], a["rows"], a["c"], a["dtype"], a["codes"], a["crs"],
                                  a["scales"], a["srs"], None)


def test_quantize_mxfp4_rejects_bad_arguments(lib):
    assert _quant(lib, dtype=2) == ENOTSUP
    assert _quant(lib, x=None) == EINVAL
    assert _quant(lib, scales=None) == EINVAL
    assert _quant(lib, c=48) == EINVAL            # MX blocks are 32 values
    assert _quant(lib, rows=0) == EINVAL
    assert _quant(lib, xrs=32) == EINVAL          # stride below the row
    assert _quant(lib, crs=16) == EINVAL          # c/2 = 32 code bytes per row
    assert _quant(lib, codes=0x200008) == EINVAL  # 16-byte stores
    assert _quant(lib, xrs=68) == EINVAL          # bf16 rows must stay 16-byte aligned


def _nr(lib, **kw):
    a = dict(x=0x100000, xrs=128, out=0x300000, ors=128, gamma=0x400000, eps=1e-6, rows=4, heads=2, c=64,
             rd=16, base=10000.0, pos0=0, step=1, dtype=1)
    a.update(kw)
    return lib.csa_norm_rope(a["x"], a["xrs"], a["out"], a["ors"], a["gamma"], a["eps"], a["rows"], a["heads"],
                             a["c"], a["rd"], a["base"], a["pos0"], a["step"], a["dtype"], None)


def test_norm_rope_rejects_bad_arguments(lib):
    assert _nr(lib, rows=0) == 0                      # nothing to do
    assert _nr(lib, dtype=2) == ENOTSUP
    assert _nr(lib, x=None) == EINVAL
    assert _nr(lib, out=None) == EINVAL
    assert _nr(lib, rows=-1) == EINVAL
    assert _nr(lib, heads=0) == EINVAL
    assert _nr(lib, rd=15) == EINVAL                  # pairs
    assert _nr(lib, rd=66) == EINVAL                  # more than c
    assert _nr(lib, eps=-1.0) == EINVAL
    assert _nr(lib, eps=float("nan")) == EINVAL
    assert _nr(lib, base=0.0) == EINVAL
    assert _nr(lib, base=float("inf")) == EINVAL
    assert _nr(lib, xrs=120) == EINVAL                # below heads * c
    assert _nr(lib, x=0x100008) == EINVAL             # 16-byte loads
    assert _nr(lib, gamma=0x400004) == EINVAL         # 16-byte gain loads
    assert _nr(lib, xrs=132) == EINVAL                # bf16 rows must stay 16-byte aligned
    assert _nr(lib, pos0=1 << 41) == EINVAL
    assert _nr(lib, pos0=(1 << 40) - 2, step=1) == EINVAL   # the last row passes the limit
    assert _nr(lib, out=0x100100) == EINVAL           # partial overlap with x
    assert _nr(lib, c=68, xrs=136, ors=136) == ENOTSUP   # bf16 c must be a multiple of 8
    assert _nr(lib, c=2056, xrs=4112, ors=4112, rd=0) == ENOTSUP   # above 2048 bf16 values
    assert _nr(lib, c=1024, xrs=2048, ors=2048, rd=514) == ENOTSUP   # at most 256 rotation pairs


def _gop(lib, **kw):
    a = dict(o=0x100000, WG=0x200000, WO=0x300000, n=300, n_h=8, c=64, g=2, d_g=128, d=320, dtype=1,
             mid=0x400000, out=0x500000)
    a.update(kw)
    return lib.csa_grouped_out_proj(a["o"], a["WG"], a["WO"], a["n"], a["n_h"], a["c"], a["g"], a["d_g"], a["d"],
                                    a["dtype"], a["mid"], a["out"], None)


def test_grouped_out_proj_rejects_bad_arguments(lib):
    assert _gop(lib, n=0) == 0                       # nothing to do
    assert _gop(lib, n=-1) == EINVAL
    assert _gop(lib, g=3) == EINVAL                  # heads do not split into 3 groups
    assert _gop(lib, d=0) == EINVAL
    assert _gop(lib, o=None) == EINVAL
    assert _gop(lib, mid=None) == EINVAL
    assert _gop(lib, WG=0x200008) == EINVAL          # 16-byte gathers
    assert _gop(lib, dtype=0) == ENOTSUP             # bf16 only
    assert _gop(lib, c=40) == ENOTSUP                # (n_h/g) c = 160: not a multiple of 64
    assert _gop(lib, d_g=100) == ENOTSUP             # g d_g = 200


def test_index_topk_workspace_size_grows_with_candidates(lib):
    small = lib.csa_index_topk_workspace_size(1, 4, 100, 8)
    big = lib.csa_index_topk_workspace_size(1, 4, 100000, 8)
    assert 0 < small < big
    assert lib.csa_index_topk_workspace_size(1, 8192, 2048, 512) >= 8192 * 2048 * 4
    assert lib.csa_index_topk_workspace_size(0, 4, 100, 8) == 0


def _attend(lib, fn="csa_attend", ws_bytes=0, **kw):
    a = dict(q=FAKE, Cc=FAKE, cbs=0, idx=FAKE, raw=FAKE, rbs=0, pos0=0, sink=FAKE, b=1, n_q=4, t0=0,
             n_comp=1, n_raw=4, n_h=2, c=8, k=2, m=4, n_win=4, scale=0.5, dtype=0, ws=None, out=FAKE)
    a.update(kw)
    if fn == "csa_attend":
        return lib.csa_attend(a["q"], a["Cc"], a["cbs"], a["idx"], a["raw"], a["rbs"], a["pos0"],
                              a["sink"], a["b"], a["n_q"], a["t0"], a["n_comp"], a["n_raw"], a["n_h"],
                              a["c"], a["k"], a["m"], a["n_win"], a["scale"], a["dtype"], a["ws"],
                              ws_bytes, a["out"], None)
    return lib.hca_attend(a["q"], a["Cc"], a["cbs"], a["raw"], a["rbs"], a["pos0"], a["sink"], a["b"],
                          a["n_q"], a["t0"], a["n_comp"], a["n_raw"], a["n_h"], a["c"], a["m"],
                          a["n_win"], a["scale"], a["dtype"], a["ws"], ws_bytes, a["out"], None)


@pytest.mark.parametrize("fn", ["csa_attend", "hca_attend"])
def test_attend_rejects_bad_arguments(lib, fn):
    assert _attend(lib, fn, q=None) == EINVAL
    assert _attend(lib, fn, sink=None) == EINVAL
    assert _attend(lib, fn, n_win=0) == EINVAL
    assert _attend(lib, fn, scale=float("nan")) == EINVAL
    # the window of queries 0..3 needs raw rows 0..3
    assert _attend(lib, fn, n_raw=3) == EINVAL
    assert _attend(lib, fn, pos0=1) == EINVAL
    assert _attend(lib, fn, t0=10, n_raw=4, pos0=7) == EINVAL
    assert _attend(lib, fn, dtype=4) == ENOTSUP
    assert _attend(lib, fn, c=2048) == ENOTSUP
    assert _attend(lib, fn, rbs=3) == EINVAL


def test_attend_norm_rope_rejects_bad_arguments(lib):
    def call(ws_bytes=0, **kw):
        a = dict(q=FAKE, gq=FAKE, eps=1e-6, rd=64, base=10000.0, Cc=FAKE, cbs=0, idx=FAKE, raw=FAKE, rbs=0,
                 pos0=0, sink=FAKE, b=1, n_q=4, t0=0, n_comp=1, n_raw=4, n_h=64, c=512, k=2, m=4, n_win=4,
                 scale=0.05, dtype=1, ws=None, out=FAKE)
        a.update(kw)
        return lib.csa_attend_norm_rope(a["q"], a["gq"], a["eps"], a["rd"], a["base"], a["Cc"], a["cbs"],
                                        a["idx"], a["raw"], a["rbs"], a["pos0"], a["sink"], a["b"], a["n_q"],
                                        a["t0"], a["n_comp"], a["n_raw"], a["n_h"], a["c"], a["k"], a["m"],
                                        a["n_win"], a["scale"], a["dtype"], a["ws"], ws_bytes, a["out"], None)
    assert call(q=None) == EINVAL
    assert call(gq=None) == EINVAL
    assert call(gq=FAKE + 4) == EINVAL          # gain not 16-byte aligned
    assert call(eps=-1.0) == EINVAL
    assert call(eps=float("inf")) == EINVAL
    assert call(rd=63) == EINVAL
    assert call(rd=-2) == EINVAL
    assert call(rd=514) == EINVAL             # more rotated dimensions than a head has
    assert call(base=0.0) == EINVAL
    assert call(base=float("nan")) == EINVAL
    assert call(n_q=1, t0=1 << 41, n_raw=4, pos0=(1 << 41) - 3) == EINVAL
    assert call(n_raw=3) == EINVAL
    assert call(k=3, idx=None) == EINVAL
    # the fused form runs on the bf16 c = 512 tile path only
    assert call(dtype=0) == ENOTSUP
    assert call(c=256) == ENOTSUP
    assert call(n_h=32, sink=FAKE) == ENOTSUP
    assert call(k=4096) == ENOTSUP
    # a split decode query needs the attention's workspace
    kw = dict(n_q=1, t0=4095, n_comp=1024, n_raw=128, pos0=3968, k=512, n_win=128)
    need = lib.csa_attend_workspace_size(1, 1, 4095, 1024, 64, 512, 512, 4, 128, 1)
    assert call(ws=None, ws_bytes=need, **kw) == EINVAL
    assert call(ws=0x100000, ws_bytes=need - 1, **kw) == ENOSPC


def test_hca_attend_norm_rope_rejects_bad_arguments(lib):
    def call(ws_bytes=0, **kw):
        a = dict(q=FAKE, gq=FAKE, eps=1e-6, rd=64, base=10000.0, Cc=FAKE, cbs=0, raw=FAKE, rbs=0, pos0=0, sink=FAKE,
                 b=1, n_q=4, t0=0, n_comp=1, n_raw=4, n_h=64, c=512, mp=4, n_win=4, scale=0.05, dtype=1, ws=None,
                 out=FAKE)
        a.update(kw)
        return lib.hca_attend_norm_rope(a["q"], a["gq"], a["eps"], a["rd"], a["base"], a["Cc"], a["cbs"], a["raw"],
                                        a["rbs"], a["pos0"], a["sink"], a["b"], a["n_q"], a["t0"], a["n_comp"],
                                        a["n_raw"], a["n_h"], a["c"], a["mp"], a["n_win"], a["scale"], a["dtype"],
                                        a["ws"], ws_bytes, a["out"], None)
    assert call(q=None) == EINVAL
    assert call(gq=None) == EINVAL
    assert call(gq=FAKE + 8) == EINVAL
    assert call(eps=float("nan")) == EINVAL
    assert call(rd=7) == EINVAL
    assert call(rd=1024) == EINVAL
    assert call(base=-1.0) == EINVAL
    assert call(n_raw=3) == EINVAL
    assert call(mp=0) == EINVAL
    assert call(dtype=0) == ENOTSUP
    assert call(c=256) == ENOTSUP
    assert call(n_h=96) == ENOTSUP
    # one query per sequence over 8192 entries splits: workspace required
    kw = dict(n_q=1, t0=8192 * 128 + 5, n_comp=8192, n_raw=128, pos0=8192 * 128 + 5 - 127, mp=128, n_win=128)
    need = lib.hca_attend_workspace_size(1, 1, 8192 * 128 + 5, 8192, 64, 512, 128, 128, 1)
    assert need > 0
    assert call(ws=None, ws_bytes=need, **kw) == EINVAL
    assert call(ws=0x100000, ws_bytes=need - 1, **kw) == ENOSPC


def test_attend_decode_needs_workspace(lib):
    # one bf16 64-head c=512 query splits its entries: scratch is required
    need = lib.csa_attend_workspace_size(1, 1, 4095, 1024, 64, 512, 512, 4, 128, 1)
    assert need > 0
    kw = dict(n_q=1, t0=4095, n_comp=1024, n_raw=128, pos0=3968, n_h=64, c=512, k=512, dtype=1,
              n_win=128)
    assert _attend(lib, ws=None, ws_bytes=need, **kw) == EINVAL
    assert _attend(lib, ws=0x100000, ws_bytes=need - 1, **kw) == ENOSPC
    # many queries: no scratch
    assert lib.csa_attend_workspace_size(1, 8192, 0, 2048, 64, 512, 512, 4, 128, 1) == 0


def test_hca_layer_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(C=FAKE, Z=FAKE, B=FAKE, q=FAKE, raw=FAKE, sink=FAKE, b=1, n=128, c=512, mp=128,
                 n_h=64, n_win=128, scale=0.1, dtype=1, Cc=FAKE, ws=0x100000, wsb=1 << 30, out=FAKE)
        a.update(kw)
        return lib.hca_layer(a["C"], a["Z"], a["B"], a["q"], a["raw"], a["sink"], a["b"], a["n"], a["c"],
                             a["mp"], a["n_h"], a["n_win"], a["scale"], a["dtype"], a["Cc"], a["ws"],
                             a["wsb"], a["out"], None)
    assert call(C=None) == EINVAL
    assert call(mp=0) == EINVAL
    assert call(dtype=3) == ENOTSUP
    # 128 queries: few enough work items that the attention splits its lists
    assert lib.hca_layer_workspace_size(1, 128, 64, 512, 128, 128, 1) > 0
    assert call(wsb=0) == ENOSPC
    assert call(Cc=None) == EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no library, no fallback: every entry point goes through load_library,
    # which raises when libcsa.so is absent
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library(str(tmp_path / "libcsa.so"))


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(8, 4)
    with pytest.raises(ValueError):
        L.csa_compress(x, x, x, x, torch.zeros(4, 4), torch.zeros(4, 4), 4)


def test_misaligned_rows_are_rejected(lib):
    # rows moved 16 bytes per lane (bf16 MFMA attention at c = 512, vector
    # compressor and indexer rows) need 16-byte aligned pointers and strides
    dec = dict(n_q=1, t0=4095, n_comp=1024, n_raw=128, pos0=3968, n_h=64, c=512, k=512, dtype=1, n_win=128,
               ws=0x100000, ws_bytes=1 << 30)
    for bad in (dict(q=FAKE + 2), dict(Cc=FAKE + 8), dict(raw=FAKE + 4), dict(out=FAKE + 2),
                dict(cbs=1024 * 512 + 1), dict(rbs=128 * 512 + 4), dict(sink=FAKE + 2)):
        kw = dict(dec)
        kw.update(bad)
        assert _attend(lib, **kw) == EINVAL, bad
        assert _attend(lib, "hca_attend", **kw) == EINVAL, bad
    # the generic float32 path reads elements one at a time: natural alignment
    assert _attend(lib, q=FAKE + 2) == EINVAL
    # compressor: c = 8 bf16 is one 16-byte vector per row
    for bad in (dict(Ca=FAKE + 2), dict(Zb=FAKE + 8), dict(out=FAKE + 4), dict(obs=4 * 8 + 1),
                dict(pCb=FAKE + 2, pZb=FAKE)):
        assert _compress(lib, dtype=1, **bad) == EINVAL, bad
    # indexer: bf16 keys of 16 dims (32 bytes per row)
    for bad in (dict(qI=FAKE + 2), dict(KI=FAKE + 16 + 2), dict(cbs=2 * 16 + 1), dict(w=FAKE + 2),
                dict(idx=FAKE + 1)):
        assert _topk(lib, dtype=1, **bad) == EINVAL, bad
    # MXFP4: code rows 16-byte aligned, 4-byte scale words
    assert _topk_mx(lib, qI=FAKE + 8) == EINVAL
    assert _topk_mx(lib, KI=FAKE + 8) == EINVAL
    assert _topk_mx(lib, cI=128, KS=FAKE + 2) == EINVAL


def test_index_topk_noalloc_rejects_before_launch(lib):
    def call(**kw):
        a = dict(qI=FAKE, w=FAKE, KI=FAKE, cbs=0, b=1, n_q=8, t0=0, n_comp=2, nh=2, cI=16, m=4, k=4,
                 dtype=0, idx=FAKE, score=None)
        a.update(kw)
        return lib.csa_index_topk_noalloc(a["qI"], a["w"], a["KI"], a["cbs"], a["b"], a["n_q"], a["t0"],
                                          a["n_comp"], a["nh"], a["cI"], a["m"], a["k"], a["dtype"], a["idx"],
                                          a["score"], None)
    # the same validation as csa_index_topk
    assert call(k=0) == EINVAL
    assert call(n_comp=3) == EINVAL
    assert call(dtype=9) == ENOTSUP
    assert call(qI=FAKE + 2, dtype=1) == EINVAL
    # 64 sequences of a 2^20-token decode need more than the 80 MiB scratch
    big = dict(b=64, n_q=1, t0=262144 * 4 - 1, n_comp=262144, nh=64, cI=128, k=512, dtype=1)
    assert lib.csa_index_topk_workspace_size(64, 1, 262144, 512) > 80 * 1024 * 1024
    assert call(**big) == ENOSPC


def test_block_pool_hands_out_and_takes_back_ids():
    pool = B.BlockPool(5)
    a = pool.alloc(3)
    assert sorted(a) == [0, 1, 2] and pool.available() == 2
    with pytest.raises(L.CsaError):
        pool.alloc(3)                      # only 2 left: nothing taken
    assert pool.available() == 2
    pool.release([a[1]])
    assert pool.alloc(1) == [a[1]]        # the last released id comes back first
    with pytest.raises(L.CsaError):
        pool.release([a[0], a[0]])         # listed twice: nothing released
    with pytest.raises(L.CsaError):
        pool.release([4])                  # never allocated
    assert pool.available() == 2
    pool.release(a)
    assert pool.available() == 5
    pool.close()
    lib = L.load_library()
    assert lib.csa_block_pool_create(0) is None
    assert lib.csa_block_pool_available(None) == -1


def test_paged_geometry_and_validation(lib):
    # m = 4, m' = 128: 32 CSA entries, 32 keys and 1 HCA entry per block
    assert lib.csa_paged_block_bytes(512, 128, 4, 128) == 2 * (32 * 512 + 32 * 128 + 512)
    assert lib.csa_paged_block_bytes(512, 128, 4, 6) == 0    # 12-token blocks: 3 CSA entries, not a power of two
    st = lib.csa_paged_state_bytes(512, 128, 4, 128, 128)
    assert st >= 2 * (2 * 128 * 512 + 6 * 4 * 512 + 6 * 4 * 128 + 2 * 128 * 512) and st % 256 == 0
    z = [FAKE] * 15
    ok = dict(state=FAKE, blocks=FAKE, nb=8, table=FAKE, bts=4, slot=None, pos=FAKE, b=2)
    def app(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.csa_paged_append(a["state"], a["blocks"], a["nb"], a["table"], a["bts"], a["slot"], a["pos"],
                                    a["b"], *z, 512, 128, 4, 128, 128, kw.get("dtype", 1), None)
    assert app(dtype=0) == ENOTSUP
    assert app(state=None) == EINVAL
    assert app(pos=FAKE + 4) == EINVAL     # int64 positions
    assert app(nb=0) == EINVAL
    # attention: c = 512 MFMA path only; the table must hold n_comp_max entries
    def att(**kw):
        a = dict(n_max=64, c=512, nh=64, k=64, dtype=1)
        a.update(kw)
        return lib.csa_paged_attend(FAKE, FAKE, 8, FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, 2, a["n_max"], a["nh"],
                                    a["c"], 128, a["k"], 4, 128, 128, 0.05, a["dtype"], FAKE, 1 << 30, FAKE, None)
    assert att(c=256) == ENOTSUP
    assert att(nh=32) == ENOTSUP
    assert att(n_max=4 * 32 + 1) == EINVAL
    assert att(dtype=0) == ENOTSUP
    # HCA: the list is split at least every 2048 entries and the split merge
    # takes at most 16384 splits: 2^25 entries with the window
    def hca(n_max, ws_bytes=1 << 30):
        return lib.hca_paged_attend(FAKE, FAKE, 8, FAKE, 1 << 26, None, FAKE, FAKE, FAKE, 2, n_max, 64, 512, 128, 4,
                                    128, 128, 0.05, 1, FAKE, ws_bytes, FAKE, None)
    assert hca((1 << 25) - 127) == ENOTSUP
    assert hca((1 << 25) - 128) == ENOSPC      # supported; its split partials need more workspace


def test_release_build_has_no_debug_checks(lib):
    # the debug entry points exist in every build; the release build
    # reports that it carries no bounds checks
    assert lib.csa_debug_enabled() == 0
    assert lib.csa_debug_set_entry_limit(10) == ENOTSUP
    assert lib.csa_strerror(-5).decode() == "bounds check failed (debug build)"


def test_debug_build_exports_and_enables_checks():
    from long_context_compressed_csa_amd import build as B
    if not os.path.exists(B.DEBUG_LIB):
        pytest.fail(f"{B.DEBUG_LIB} is missing: the build makes it beside libcsa.so")
    dbg = L._binding.open_library(B.DEBUG_LIB)
    assert dbg.csa_debug_enabled() == 1
    assert dbg.csa_debug_set_entry_limit(-1) == EINVAL
