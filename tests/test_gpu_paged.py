"""GPU parity of the heterogeneous decode cache (paged blocks + state cache)
against the oracle's per-request decode states.

Four request slots share one block pool; requests join the batch at
different steps, so every decode step mixes lengths (variable-length
batching), batch rows map to slots in a permuted order, and blocks come from
the library's block pool interleaved across requests (no request's blocks
are contiguous).  Every step appends each active request's token
(csa_paged_append: state update, CSA/indexer entries every 4 tokens, HCA
entries every 128); at check steps the CSA indexer (csa_paged_index_topk),
CSA attention (csa_paged_attend) and HCA attention (hca_paged_attend) run on
the whole batch and are compared with the oracle computed from the same
tokens alone, with compressed entries stored in bf16 (the cache's storage).
"""

import math
import sys

import numpy as np
import pytest
import torch

import long_context_compressed_csa_amd as L
import oracle as O
from parity_helpers import assert_close, assert_index_sets, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _bf16(a):
    return to64(torch.tensor(np.asarray(a), dtype=torch.float32).to(torch.bfloat16))


def test_paged_decode_mixed_lengths_matches_oracle():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    L.load_library()
    c, cI, m, mp, nw, nh, nI, k = 512, 128, 4, 128, 128, 64, 64, 96
    scale = 1.0 / math.sqrt(c)
    T = 520
    admit = [0, 37, 300, 5]          # step at which each slot's request starts
    slots = len(admit)
    checks = {40, 131, 259, 303, 306, T - 1}
    say(f"paged decode: {slots} requests admitted at {admit}, {T} steps, checks at {sorted(checks)}")
    gen = torch.Generator().manual_seed(91)
    rnd = lambda *s: (torch.randn(s, generator=gen) / math.sqrt(s[-1])).to(torch.bfloat16)
    biases = {"Ba": rnd(m, c), "Bb": rnd(m, c), "IBa": rnd(m, cI), "IBb": rnd(m, cI), "B_h": rnd(mp, c)}
    sink = torch.randn(nh, generator=gen)
    gb = {x: v.to(DEV) for x, v in biases.items()}
    ob = {x: to64(v) for x, v in biases.items()}
    ob_csa = {"Ba": ob["Ba"], "Bb": ob["Bb"], "IBa": ob["IBa"], "IBb": ob["IBb"]}

    n_blocks, bt_stride = 40, 8
    cache = L.PagedCache(n_blocks, slots, bt_stride, c, cI, m, mp, nw, device=DEV)
    cache.blocks.fill_(float("nan"))     # nothing unwritten may be read
    cache.state.fill_(float("nan"))
    pool = L.BlockPool(n_blocks)
    pool.alloc(3)                          # a few ids held elsewhere: the requests' ids are scattered
    table = torch.zeros((slots, bt_stride), dtype=torch.int32)
    csa_o = [O.CsaDecodeState(m=m, n_win=nw, c=c, c_I=cI) for _ in range(slots)]
    hca_o = [O.HcaDecodeState(m_prime=mp, n_win=nw) for _ in range(slots)]
    ws_i = torch.empty(max(L.load_library().csa_index_topk_workspace_size(slots, 1, 4096, k), 256),
                       dtype=torch.uint8, device=DEV)
    n_checked = n_ties = 0
    for step in range(T):
        active = [r for r in range(slots) if step >= admit[r]]
        order = active[::-1]               # batch row i -> request slot order[i]
        pos = [step - admit[r] for r in order]
        # a block for every request whose token opens a new 128-token block
        for r, t in zip(order, pos):
            if t % (m * mp // math.gcd(m, mp)) == 0:
                table[r, t // 128] = pool.alloc(1)[0]
        cache.table.copy_(table)
        tok = {x: rnd(len(order), c) for x in ("Ca", "Cb", "Za", "Zb", "C_h", "Z_h")}
        tok.update({x: rnd(len(order), cI) for x in ("ICa", "ICb", "IZa", "IZb")})
        g_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
        g_slot = torch.tensor(order, dtype=torch.int32, device=DEV)
        L.csa_paged_append(cache, g_pos, {x: v.to(DEV) for x, v in tok.items()}, gb, req_slot=g_slot)
        for i, r in enumerate(order):
            csa_o[r].append({x: to64(tok[x][i]) for x in ("Ca", "Cb", "Za", "Zb", "ICa", "ICb", "IZa", "IZb")},
                            ob_csa)
            hca_o[r].append(to64(tok["C_h"][i]), to64(tok["Z_h"][i]), ob["B_h"])
        if step not in checks:
            continue
        torch.cuda.synchronize()
        b = len(order)
        q = rnd(b, nh, c)
        qI = rnd(b, nI, cI)
        w = torch.nn.functional.softplus(torch.randn((b, nI), generator=gen))
        n_comp_max = max((t + 1) // m for t in pos)
        n_hca_max = max((t + 1) // mp for t in pos)
        idx = L.csa_paged_index_topk(cache, qI.to(DEV), w.to(DEV), g_pos, n_comp_max, k, req_slot=g_slot,
                                     workspace=ws_i)
        out = L.csa_paged_attend(cache, q.to(DEV), idx, sink.to(DEV), g_pos, n_comp_max, scale, req_slot=g_slot)
        h_out = L.hca_paged_attend(cache, q.to(DEV), sink.to(DEV), g_pos, n_hca_max, scale, req_slot=g_slot)
        torch.cuda.synchronize()
        oidx = np.full((b, k), -1, dtype=np.int64)
        for i, (r, t) in enumerate(zip(order, pos)):
            st, hs = csa_o[r], hca_o[r]
            assert st.t == t and hs.t == t
            Cc16 = _bf16(np.array(st.Ccomp).reshape(-1, c))
            KI16 = _bf16(np.array(st.KIcomp).reshape(-1, cI))
            nc = Cc16.shape[0]
            sc = O.index_scores(to64(qI[i])[None], to64(w[i])[None], KI16, [t], m)
            oi = O.topk_select(sc[0], nc, k)
            oidx[i] = oi
            n_ties += assert_index_sets(idx[i:i + 1].cpu().numpy(), oi[None], sc, [nc], k, f"step {step} slot {r}")
            raw = np.stack([row for _, row in st.window])
            want = O.csa_attend(to64(q[i])[None], Cc16, oi[None], raw, st.window[0][0], to64(sink), [t], nw, scale, m)
            if set(idx[i].cpu().numpy().tolist()) == set(oi.tolist()):
                assert_close(out[i], want[0], torch.bfloat16, f"step {step} slot {r} csa (chained)")
            # the cache contents: entries, keys and HCA entries in the request's blocks
            E1 = 32
            for s in sorted({0, nc // 2, nc - 1} - {-1}):
                if nc == 0:
                    break
                blk = int(table[r, s // E1])
                base = blk * cache.block_bytes // 2
                got_e = cache.blocks[base + (s % E1) * c: base + (s % E1 + 1) * c]
                got_k = cache.blocks[base + E1 * c + (s % E1) * cI: base + E1 * c + (s % E1 + 1) * cI]
                assert_close(got_e[None], np.array(st.Ccomp[s])[None], torch.bfloat16, f"slot {r} entry {s}")
                assert_close(got_k[None], np.array(st.KIcomp[s])[None], torch.bfloat16, f"slot {r} key {s}")
            H16 = _bf16(np.array(hs.entries).reshape(-1, c))
            hraw = np.stack([row for _, row in hs.window])
            hwant = O.hca_attend(to64(q[i])[None], H16, hraw, hs.window[0][0], to64(sink), [t], mp, nw, scale)
            assert_close(h_out[i], hwant[0], torch.bfloat16, f"step {step} slot {r} hca")
            for s in range(H16.shape[0]):
                blk = int(table[r, s])
                base = blk * cache.block_bytes // 2 + E1 * (c + cI)
                assert_close(cache.blocks[base: base + c][None], np.array(hs.entries[s])[None], torch.bfloat16,
                             f"slot {r} hca entry {s}")
            n_checked += 1
        # the attention step on the oracle's selection, every row
        out_o = L.csa_paged_attend(cache, q.to(DEV), torch.tensor(oidx, dtype=torch.int32, device=DEV),
                                   sink.to(DEV), g_pos, n_comp_max, scale, req_slot=g_slot)
        torch.cuda.synchronize()
        for i, (r, t) in enumerate(zip(order, pos)):
            st = csa_o[r]
            Cc16 = _bf16(np.array(st.Ccomp).reshape(-1, c))
            raw = np.stack([row for _, row in st.window])
            want = O.csa_attend(to64(q[i])[None], Cc16, oidx[i][None], raw, st.window[0][0], to64(sink), [t], nw,
                                scale, m)
            assert_close(out_o[i], want[0], torch.bfloat16, f"step {step} slot {r} csa (oracle selection)")
    print(f"[paged] {n_checked} (step, request) checks, {n_ties} selections settled a near-tie differently",
          flush=True)
    assert n_checked >= 15
    pool.close()


def test_hca_paged_attend_many_splits_matches_oracle():
    """A paged HCA list long enough for more splits than one wave has lanes:
    140,000 entries plus the window take 69 splits (one per 2048 entries), so
    the split merge reads some splits' (maximum, sum) in a second round.  The
    pool is filled with random entries, the request's last block is appended
    token by token (its HCA entry, and the window ring, written by the
    library), and the oracle attends over the entries read back from the
    pool."""
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    L.load_library()
    c, cI, m, mp, nw, nh = 512, 128, 4, 128, 128, 64
    scale = 1.0 / math.sqrt(c)
    n_prior = 139_999                   # HCA entries already in the pool
    n_blocks = n_prior + 1              # one block per 128 tokens
    P0 = mp * n_prior                   # first token of the last block
    t = P0 + mp - 1                     # the query: the last block complete
    n_vis = (t + 1) // mp               # 140,000 entries
    say(f"paged HCA, {n_vis} entries + {nw} window rows, t = {t}")
    cache = L.PagedCache(n_blocks, 1, n_blocks, c, cI, m, mp, nw, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    cache.blocks.normal_(0.0, 1.0 / math.sqrt(c), generator=g)
    cache.state.zero_()
    perm = torch.randperm(n_blocks, generator=g, device=DEV).to(torch.int32)
    cache.table[0].copy_(perm)
    gen = torch.Generator().manual_seed(18)
    rnd = lambda *s: (torch.randn(s, generator=gen) / math.sqrt(s[-1])).to(torch.bfloat16)
    biases = {"Ba": rnd(m, c), "Bb": rnd(m, c), "IBa": rnd(m, cI), "IBb": rnd(m, cI), "B_h": rnd(mp, c)}
    gb = {x: v.to(DEV) for x, v in biases.items()}
    slot = torch.zeros(1, dtype=torch.int32, device=DEV)
    window = []
    for p in range(P0, t + 1):
        tok = {x: rnd(1, c) for x in ("Ca", "Cb", "Za", "Zb", "C_h", "Z_h")}
        tok.update({x: rnd(1, cI) for x in ("ICa", "ICb", "IZa", "IZb")})
        L.csa_paged_append(cache, torch.tensor([p], dtype=torch.int64, device=DEV),
                           {x: v.to(DEV) for x, v in tok.items()}, gb, req_slot=slot)
        window.append(to64(tok["C_h"][0]))
    q = rnd(1, nh, c)
    sink = torch.randn(nh, generator=gen)
    out = L.hca_paged_attend(cache, q.to(DEV), sink.to(DEV), torch.tensor([t], dtype=torch.int64, device=DEV),
                             n_vis, scale, req_slot=slot)
    torch.cuda.synchronize()
    # entry s sits in block table[s], after the block's 32 CSA entries and 32 keys
    rows = cache.blocks.view(n_blocks, cache.block_bytes // 2)
    off = 32 * (c + cI)
    H = to64(rows[perm[:n_vis].long(), off: off + c].cpu())
    want = O.hca_attend(to64(q[0])[None], H, np.stack(window), P0, to64(sink), [t], mp, nw, scale)
    assert_close(out[0], want[0], torch.bfloat16, "paged HCA, 69 splits")
    del cache, rows
    torch.cuda.empty_cache()
