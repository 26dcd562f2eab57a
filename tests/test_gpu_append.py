"""Paged K/V append on the GPU against the oracle's append, bit for bit, and
a forward over appended rows against the oracle's attention."""

import pytest
import torch

import oracle
from workload import custom, generate
from workload.generate import Inputs

import gpu_helpers as H
from gqa_attention_agentic_amd import _lib

pytestmark = pytest.mark.gpu


def _pool_case(dtype, page_size, seed):
    g = torch.Generator().manual_seed(seed)
    H_kv, d, n_pages = 2, 128, 40
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_pages = torch.randn(n_pages, H_kv, page_size, d, generator=g).to(tdt)
    v_pages = torch.randn(n_pages, H_kv, page_size, d, generator=g).to(tdt)
    perm = torch.randperm(n_pages, generator=g).tolist()
    # branches: (existing private tokens, rows appended)
    spec = [(0, 1), (5, page_size - 5), (page_size, 2 * page_size + 3), (7, 0), (3 * page_size - 1, 1)]
    max_pages = max(-(-(a + n) // page_size) for a, n in spec) + 1
    table = torch.full((len(spec), max_pages), -1, dtype=torch.int32)
    nxt = 0
    for b, (a, n) in enumerate(spec):
        for lp in range(-(-(a + n) // page_size)):
            table[b, lp] = perm[nxt]
            nxt += 1
    rows = sum(n for _, n in spec)
    k_new = torch.randn(rows, H_kv, d, generator=g).to(tdt)
    v_new = torch.randn(rows, H_kv, d, generator=g).to(tdt)
    return k_pages, v_pages, table, [a for a, _ in spec], [n for _, n in spec], k_new, v_new


@pytest.mark.parametrize("dtype,page_size", [("bf16", 16), ("bf16", 12), ("fp32", 16), ("fp32", 5)])
def test_append_bitwise_matches_oracle(dtype, page_size):
    kp, vp, table, plen, n_new, kn, vn = _pool_case(dtype, page_size, 41 + page_size)
    ref_k, ref_v = oracle.append_kv(kp, vp, table, plen, n_new, kn, vn, page_size)
    H.say(f"[append] {dtype} ps={page_size} rows={kn.shape[0]}")
    h = H.handle_for(custom("pool", dtype=dtype, H_q=4, H_kv=2, d=128, page_size=page_size))
    gk, gv, gt = kp.cuda(), vp.cuda(), table.cuda()
    h.append_kv(kn.cuda(), vn.cuda(), gk, gv, gt, plen, n_new)
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), ref_k) and torch.equal(gv.cpu(), ref_v)


def test_append_skips_rows_whose_page_is_outside_the_pool():
    kp, vp, table, plen, n_new, kn, vn = _pool_case("bf16", 16, 7)
    bad = table.clone()
    bad[2, 1] = kp.shape[0] + 3          # a page id past the pool
    ref_k, ref_v = oracle.append_kv(kp, vp, table, plen, n_new, kn, vn, 16)
    h = H.handle_for(custom("pool", H_q=4, H_kv=2, d=128, page_size=16))
    gk, gv = kp.cuda(), vp.cuda()
    h.append_kv(kn.cuda(), vn.cuda(), gk, gv, bad.cuda(), plen, n_new)
    torch.cuda.synchronize()
    page = int(table[2, 1])
    # every slot of the page the bad entry stood for keeps its old value; the rest is appended
    assert torch.equal(gk.cpu()[page], kp[page]) and torch.equal(gv.cpu()[page], vp[page])
    keep = [p for p in range(kp.shape[0]) if p != page]
    assert torch.equal(gk.cpu()[keep], ref_k[keep]) and torch.equal(gv.cpu()[keep], ref_v[keep])


def test_append_rejects_rows_past_the_page_table():
    kp, vp, table, plen, n_new, kn, vn = _pool_case("bf16", 16, 9)
    h = H.handle_for(custom("pool", H_q=4, H_kv=2, d=128, page_size=16))
    n_new = list(n_new)
    n_new[0] = table.shape[1] * 16 + 1
    kn = torch.zeros(sum(n_new), 2, 128, dtype=torch.bfloat16)
    with pytest.raises(_lib.GqaError) as e:
        h.append_kv(kn.cuda(), kn.cuda(), kp.cuda(), vp.cuda(), table.cuda(), plen, n_new)
    assert "exceed" in str(e.value)


def test_forward_over_appended_rows():
    """Continuation: the last rows of each branch's private suffix arrive by
    append (pool slots cleared first), then the forward attends to them."""
    w = custom("append_forward", shared=(300,), branches=((0, 6, 40), (0, 9, 37)), seed=119)
    inp = generate(w, "cuda")
    ref = H.oracle_rows(w, inp)
    n_new = [6, 9]
    keep = [L - n for L, n in zip(inp.branch_private_len, n_new)]
    ks, vs = [], []
    kp, vp = inp.k_pages.clone(), inp.v_pages.clone()
    for b, (k0, n) in enumerate(zip(keep, n_new)):
        for i in range(n):
            page = int(inp.page_table[b][(k0 + i) // w.page_size])
            slot = (k0 + i) % w.page_size
            ks.append(kp[page, :, slot].clone())
            vs.append(vp[page, :, slot].clone())
            kp[page, :, slot] = 0
            vp[page, :, slot] = 0
    h = H.handle_for(w)
    h.append_kv(torch.stack(ks), torch.stack(vs), kp, vp, inp.page_table, keep, n_new)
    inp2 = Inputs(inp.q, inp.k_shared, inp.v_shared, kp, vp, inp.page_table, inp.group_shared_start,
                  inp.group_shared_len, inp.branch_group, inp.branch_q_len, inp.branch_private_len)
    o, lse, _ = H.run_library(w, inp2, handle=h)
    H.compare(w, o, lse, ref[0], ref[1], ref[2], label="forward after append")


def test_repeated_and_changed_row_lists():
    """The row list is reused while (private_len, n_new) stay the same: a
    second append with the same lengths but other rows and another page
    table, then one with other lengths, each match the oracle."""
    h = H.handle_for(custom("pool", H_q=4, H_kv=2, d=128, page_size=16))
    for seed, shift in ((51, 0), (52, 0), (53, 1)):
        kp, vp, table, plen, n_new, kn, vn = _pool_case("bf16", 16, seed)
        plen = [a + shift for a in plen]
        n_new = [max(0, n - shift) for n in n_new]
        kn, vn = kn[:sum(n_new)].contiguous(), vn[:sum(n_new)].contiguous()
        ref_k, ref_v = oracle.append_kv(kp, vp, table, plen, n_new, kn, vn, 16)
        gk, gv = kp.cuda(), vp.cuda()
        h.append_kv(kn.cuda(), vn.cuda(), gk, gv, table.cuda(), plen, n_new)
        torch.cuda.synchronize()
        assert torch.equal(gk.cpu(), ref_k) and torch.equal(gv.cpu(), ref_v), seed
