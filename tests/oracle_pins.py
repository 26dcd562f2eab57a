"""Pins that tie the fp64 oracle to facts other than itself.

Each pin raises AssertionError when the oracle disagrees with what the
pages and the mathematics fix. ``test_oracle_pins.py`` runs them on the
oracle as written, and again with plausible mistakes planted in it (on the
CPU), checking that every planted mistake makes at least one pin fail.
"""

from __future__ import annotations

import json
import math
import os
import random
from fractions import Fraction

import torch
import torch.nn.functional as F

import oracle
from oracle import fp64 as OA
from workload import custom, generate, get_workload
from workload.generate import Inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F64 = torch.float64


# ------------------------------------------------------------------ helpers --
def _parse(expr: str) -> float:
    expr = expr.strip()
    if expr.startswith("ln "):
        return math.log(float(Fraction(expr[3:])))
    return float(Fraction(expr))


def golden_inputs(g) -> Inputs:
    t = lambda x: torch.tensor(x, dtype=F64)
    starts, acc = [], 0
    for s in g["group_shared_len"]:
        starts.append(acc)
        acc += s
    return Inputs(t(g["q"]), t(g["k_shared"]), t(g["v_shared"]), t(g["k_pages"]),
                  t(g["v_pages"]), torch.tensor(g["page_table"], dtype=torch.int32),
                  starts, list(g["group_shared_len"]), list(g["branch_group"]),
                  list(g["branch_q_len"]), list(g["branch_private_len"]))


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_oracle(w, inp, **kw):
    return oracle.attention(inp, w.num_kv_heads, w.page_size, w.causal, **kw)


def q_begin_of(inp):
    out, acc = [], 0
    for t in inp.branch_q_len:
        out.append(acc)
        acc += t
    return out


def context_by_walk(inp, b, page_size):
    """Branch context assembled element by element in plain Python: a walk
    over the shared prefix, then over the page table (independent of the
    oracle's tensor gathers)."""
    g = inp.branch_group[b]
    s0, sl = inp.group_shared_start[g], inp.group_shared_len[g]
    H_kv = inp.k_shared.shape[0]
    ks, vs = [], []
    for j in range(sl):
        ks.append([inp.k_shared[kv, s0 + j].double().tolist() for kv in range(H_kv)])
        vs.append([inp.v_shared[kv, s0 + j].double().tolist() for kv in range(H_kv)])
    table = inp.page_table[b].tolist()
    for i in range(inp.branch_private_len[b]):
        page = table[i // page_size]
        slot = i - (i // page_size) * page_size
        ks.append([inp.k_pages[page, kv, slot].double().tolist() for kv in range(H_kv)])
        vs.append([inp.v_pages[page, kv, slot].double().tolist() for kv in range(H_kv)])
    return ks, vs


# ------------------------------------------------------------------- pins ---
def pin_golden_weights_123():
    g = load_golden("weights_123.json")
    inp = golden_inputs(g)
    o, lse = oracle.attention(inp, g["num_kv_heads"], g["page_size"], g["causal"])
    exp_o = [_parse(x) for x in g["expected_o"]["token_0_head_0"]]
    assert torch.allclose(o[0, 0], torch.tensor(exp_o, dtype=F64), atol=1e-12, rtol=0), (o, exp_o)
    assert abs(lse[0, 0].item() - _parse(g["expected_lse"]["token_0_head_0"])) < 1e-12, lse


def pin_golden_paged_causal():
    g = load_golden("paged_causal_uniform.json")
    inp = golden_inputs(g)
    o, lse = oracle.attention(inp, g["num_kv_heads"], g["page_size"], g["causal"])
    for t in range(3):
        exp_o = torch.tensor([_parse(x) for x in g["expected_o"][f"token_{t}"]], dtype=F64)
        exp_l = _parse(g["expected_lse"][f"token_{t}"])
        for h in range(g["num_q_heads"]):
            assert torch.allclose(o[t, h], exp_o, atol=1e-12, rtol=0), (t, h, o[t, h], exp_o)
            assert abs(lse[t, h].item() - exp_l) < 1e-12, (t, h, lse[t, h], exp_l)


def pin_golden_merge():
    g = load_golden("merge_two_shards.json")
    st = lambda s: (torch.tensor([s["m"]], dtype=F64), torch.tensor([s["l"]], dtype=F64),
                    torch.tensor([s["o"]], dtype=F64))
    for a, b in ((g["a"], g["b"]), (g["b"], g["a"])):
        m, l, o = oracle.merge_states(st(a), st(b))
        assert abs(m.item() - _parse(g["expected_merged"]["m"])) < 1e-12
        assert abs(l.item() - _parse(g["expected_merged"]["l"])) < 1e-12
        assert abs(o[0, 0].item() - _parse(g["expected_merged"]["o"][0])) < 1e-12
        on, lse = oracle.finalize((m, l, o))
        assert abs(on[0, 0].item() - _parse(g["expected_final"]["o"][0])) < 1e-12
        assert abs(lse.item() - _parse(g["expected_final"]["lse"])) < 1e-12


def pin_brute_force_tiny():
    """Pure-Python loops with math.fsum / math.exp on the tiny fp32 fan-out."""
    w = get_workload("tiny_fp32_fanout")
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    G = w.group_size
    scale = 1.0 / math.sqrt(w.head_dim)
    qb = q_begin_of(inp)
    for b in range(len(w.branches)):
        ks, vs = context_by_walk(inp, b, w.page_size)
        C, T = len(ks), inp.branch_q_len[b]
        for t in range(T):
            tok = qb[b] + t
            pos = C - T + t
            for h in range(w.num_q_heads):
                kv = h // G
                q = inp.q[tok, h].double().tolist()
                z = []
                for j in range(C):
                    if w.causal and j > pos:
                        continue
                    z.append((j, scale * math.fsum(q[c] * ks[j][kv][c] for c in range(w.head_dim))))
                m = max(s for _, s in z)
                e = [(j, math.exp(s - m)) for j, s in z]
                l = math.fsum(x for _, x in e)
                out = [math.fsum(x * vs[j][kv][c] for j, x in e) / l for c in range(w.head_dim)]
                assert torch.allclose(o[tok, h], torch.tensor(out, dtype=F64), atol=1e-12, rtol=0), (b, t, h)
                assert abs(lse[tok, h].item() - (m + math.log(l))) < 1e-12


def _sdpa_check(w, inp):
    o, lse = run_oracle(w, inp)
    G = w.group_size
    qb = q_begin_of(inp)
    scale = 1.0 / math.sqrt(w.head_dim)
    for b in range(len(w.branches)):
        T = inp.branch_q_len[b]
        if T == 0:
            continue
        ks, vs = context_by_walk(inp, b, w.page_size)
        kb = torch.tensor(ks, dtype=F64)      # [C, H_kv, d]
        vb = torch.tensor(vs, dtype=F64)
        C = kb.shape[0]
        q = inp.q[qb[b]:qb[b] + T].double().permute(1, 0, 2).unsqueeze(0)      # [1, H_q, T, d]
        k = kb.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)        # [1, H_q, C, d]
        v = vb.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
        qpos = torch.arange(C - T, C).view(-1, 1)
        kpos = torch.arange(C).view(1, -1)
        mask = (kpos <= qpos) if w.causal else torch.ones(T, C, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask)[0].permute(1, 0, 2)
        assert torch.allclose(o[qb[b]:qb[b] + T], ref, atol=1e-12, rtol=0), b
        z = (q @ k.transpose(-1, -2)) * scale
        z = z.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(z, dim=-1)[0].permute(1, 0)
        assert torch.allclose(lse[qb[b]:qb[b] + T], ref_lse, atol=1e-12, rtol=0), b


def pin_library_sdpa():
    """torch.nn.functional.scaled_dot_product_attention (fp64, CPU) with
    K/V repeated per query head and an explicit boolean mask."""
    _sdpa_check(get_workload("tiny_fp32_fanout"), generate(get_workload("tiny_fp32_fanout"), "cpu"))
    w = custom("sdpa_small", H_q=8, H_kv=2, d=32, page_size=8, shared=(40, 0),
               branches=((0, 3, 21), (0, 6, 9), (1, 1, 30), (1, 4, 4)), seed=7)
    _sdpa_check(w, generate(w, "cpu"))


def pin_closed_form_zero_q():
    """q = 0: every visible key weighs the same, so O is the mean of the
    visible V rows and LSE = ln(number of visible keys)."""
    w = custom("zero_q", H_q=4, H_kv=2, d=16, page_size=4, shared=(13,),
               branches=((0, 3, 7), (0, 5, 5), (0, 2, 0)), seed=3, causal=True)
    inp = generate(w, "cpu")
    inp.q.zero_()
    o, lse = run_oracle(w, inp)
    qb = q_begin_of(inp)
    for b in range(len(w.branches)):
        ks, vs = context_by_walk(inp, b, w.page_size)
        vb = torch.tensor(vs, dtype=F64)
        C, T = len(ks), inp.branch_q_len[b]
        for t in range(T):
            pos = C - T + t
            for h in range(w.num_q_heads):
                kv = h // w.group_size
                assert torch.allclose(o[qb[b] + t, h], vb[:pos + 1, kv].mean(0), atol=1e-12, rtol=0)
                assert abs(lse[qb[b] + t, h].item() - math.log(pos + 1)) < 1e-12


def pin_closed_form_prefill_row0():
    """Causal prefill: token 0 sees only key 0, so O = V[0] exactly and
    LSE = its scaled score."""
    w = custom("prefill", H_q=4, H_kv=2, d=16, shared=(9,), branches=((0, 9, 0),), seed=5)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    for h in range(4):
        kv = h // 2
        assert torch.equal(o[0, h], inp.v_shared[kv, 0].double())
        z = (inp.q[0, h].double() @ inp.k_shared[kv, 0].double()) / math.sqrt(16)
        assert abs(lse[0, h].item() - z.item()) < 1e-12


def pin_closed_form_dominant_key():
    """q = c * k_j for a visible key j and large c: softmax puts all its
    mass on j, so O = V[j]."""
    w = custom("dominant", H_q=2, H_kv=1, d=64, page_size=4, shared=(20,),
               branches=((0, 2, 11),), seed=9)
    inp = generate(w, "cpu")
    ks, vs = context_by_walk(inp, 0, w.page_size)
    C = len(ks)
    targets = [(0, 3, 0), (1, 24, 1)]            # (token, key j, head)
    for tok, j, h in targets:
        inp.q[tok, h] = torch.tensor(ks[j][0], dtype=inp.q.dtype) * 50.0
    o, _ = run_oracle(w, inp)
    for tok, j, h in targets:
        assert torch.allclose(o[tok, h], torch.tensor(vs[j][0], dtype=F64), atol=1e-10, rtol=0), (tok, j)


def pin_invariant_batching():
    """Combined-Q batching: a branch computed inside its group equals the
    branch computed alone (AHBM Agentic Runtime Architecture, §1.3, §3.2)."""
    w = custom("batch", H_q=4, H_kv=2, d=16, page_size=4, shared=(17,),
               branches=((0, 3, 6), (0, 2, 9), (0, 4, 4)), seed=13)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    qb = q_begin_of(inp)
    for b in range(3):
        T = inp.branch_q_len[b]
        alone = Inputs(inp.q[qb[b]:qb[b] + T], inp.k_shared, inp.v_shared, inp.k_pages,
                       inp.v_pages, inp.page_table[b:b + 1], inp.group_shared_start,
                       inp.group_shared_len, [0], [T], [inp.branch_private_len[b]])
        o1, l1 = run_oracle(w, alone)
        assert torch.equal(o1, o[qb[b]:qb[b] + T]) and torch.equal(l1, lse[qb[b]:qb[b] + T])


def _shard_partition(kind, C, rng):
    idx = list(range(C))
    if kind == "contiguous":
        n = rng.randint(2, 6)
        cuts = sorted(rng.sample(range(1, C), min(n - 1, C - 1)))
        bounds = [0] + cuts + [C]
        return [idx[bounds[i]:bounds[i + 1]] for i in range(len(bounds) - 1)]
    if kind == "round_robin":
        # ADR-0060, §2.1-§2.2: token i lives on PE (start_pe + i) mod N.
        N, start = 8, rng.randint(0, 7)
        return [[i for i in idx if (start + i) % N == pe] for pe in range(N)]
    if kind == "with_empty":
        parts = _shard_partition("contiguous", C, rng)
        return parts[:1] + [[]] + parts[1:] + [[]]
    raise ValueError(kind)


def pin_invariant_split_merge():
    """Split-KV + merge equals unsplit attention for any partition of the
    keys, any merge order and any tree (ADR-0060, §4; AHBM Agentic Runtime
    Architecture, §3.4-§3.5 hierarchical reduction), and one shard reduces
    to O / l (ADR-0060, §0.5.4, N = 1)."""
    w = custom("split", H_q=4, H_kv=2, d=16, page_size=4, shared=(29,),
               branches=((0, 4, 11), (0, 2, 6)), seed=17)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    rng = random.Random(0)
    qb = q_begin_of(inp)
    scale = 1.0 / math.sqrt(w.head_dim)
    for b in range(2):
        kb, vb = oracle.branch_context(inp, b, w.page_size)
        C, T = kb.shape[0], inp.branch_q_len[b]
        rowpos = torch.arange(C - T, C)
        for h in range(w.num_q_heads):
            kv = h // w.group_size
            qr = inp.q[qb[b]:qb[b] + T, h].double()
            ref_o, ref_l = o[qb[b]:qb[b] + T, h], lse[qb[b]:qb[b] + T, h]
            one = oracle.finalize(oracle.partial_state(qr, kb[:, kv], vb[:, kv], torch.arange(C),
                                                       rowpos, w.causal, scale))
            assert torch.allclose(one[0], ref_o, atol=1e-13, rtol=0)
            assert torch.allclose(one[1], ref_l, atol=1e-13, rtol=0)
            for kind in ("contiguous", "round_robin", "with_empty"):
                parts = _shard_partition(kind, C, rng)
                states = []
                for p in parts:
                    pi = torch.tensor(p, dtype=torch.int64)
                    states.append(oracle.partial_state(qr, kb[pi, kv], vb[pi, kv], pi, rowpos,
                                                       w.causal, scale))
                rng.shuffle(states)
                acc = states[0]
                for s in states[1:]:
                    acc = oracle.merge_states(acc, s)
                fo, fl = oracle.finalize(acc)
                assert torch.allclose(fo, ref_o, atol=1e-12, rtol=0), kind
                assert torch.allclose(fl, ref_l, atol=1e-12, rtol=0), kind
    # hierarchical 32 -> 8 -> 4 -> 1 equals the flat fold
    b, h = 0, 1
    kb, vb = oracle.branch_context(inp, b, w.page_size)
    C, T = kb.shape[0], inp.branch_q_len[b]
    qr = inp.q[:T, h].double()
    rowpos = torch.arange(C - T, C)
    chunks = [list(range(i, C, 32)) for i in range(32)]
    kv = h // w.group_size
    states = [oracle.partial_state(qr, kb[torch.tensor(c, dtype=torch.int64), kv],
                                   vb[torch.tensor(c, dtype=torch.int64), kv],
                                   torch.tensor(c, dtype=torch.int64), rowpos, w.causal, scale)
              for c in chunks]
    level = states
    for width in (4, 2, 8):
        nxt = []
        for i in range(0, len(level), width):
            acc = level[i]
            for s in level[i + 1:i + width]:
                acc = oracle.merge_states(acc, s)
            nxt.append(acc)
        level = nxt
    assert len(level) == 1
    fo, fl = oracle.finalize(level[0])
    assert torch.allclose(fo, o[:T, h], atol=1e-12, rtol=0)
    assert torch.allclose(fl, lse[:T, h], atol=1e-12, rtol=0)


def pin_invariant_causal():
    """Changing a key after a row's position leaves that row unchanged;
    changing a visible key changes it (ADR-0060, §5.4)."""
    w = custom("causal", H_q=2, H_kv=1, d=16, page_size=4, shared=(10,),
               branches=((0, 4, 6),), seed=19)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    # context 16, queries at positions 12..15; key 14 is private token 4 (page 1, slot 0)
    page = inp.page_table[0, 1].item()
    inp.k_pages[page, 0, 0] += 3.0
    inp.v_pages[page, 0, 0] -= 2.0
    o2, lse2 = run_oracle(w, inp)
    assert torch.equal(o2[:2], o[:2]) and torch.equal(lse2[:2], lse[:2])   # positions 12, 13
    assert not torch.allclose(o2[2:], o[2:], atol=1e-6)                    # positions 14, 15


def pin_invariant_gqa_map():
    """Perturbing KV head kv changes exactly query heads kv*G .. kv*G+G-1."""
    w = custom("gqa", H_q=6, H_kv=3, d=16, page_size=4, shared=(12,),
               branches=((0, 2, 5),), seed=23)
    inp = generate(w, "cpu")
    o, _ = run_oracle(w, inp)
    inp.k_shared[1] += 1.0
    inp.v_shared[1] *= 2.0
    o2, _ = run_oracle(w, inp)
    for h in range(6):
        changed = not torch.allclose(o2[:, h], o[:, h], atol=1e-9)
        assert changed == (h in (2, 3)), h


def pin_invariant_paging():
    """Pages are referenced, not copied (AHBM Agentic Runtime Architecture,
    §3.1): renumbering the physical pages (table rewritten) changes nothing,
    and a prefix copied into every branch's private pages gives the same
    result as the shared prefix."""
    w = custom("paging", H_q=4, H_kv=2, d=16, page_size=4, shared=(12,),
               branches=((0, 3, 9), (0, 2, 5)), seed=29)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    n = inp.k_pages.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1))
    new_k = torch.empty_like(inp.k_pages)
    new_v = torch.empty_like(inp.v_pages)
    new_k[perm] = inp.k_pages
    new_v[perm] = inp.v_pages
    table = inp.page_table.clone()
    valid = table >= 0
    table[valid] = perm[table[valid].long()].int()
    inp2 = Inputs(inp.q, inp.k_shared, inp.v_shared, new_k, new_v, table,
                  inp.group_shared_start, inp.group_shared_len, inp.branch_group,
                  inp.branch_q_len, inp.branch_private_len)
    o2, l2 = run_oracle(w, inp2)
    assert torch.equal(o2, o) and torch.equal(l2, lse)
    # copy the 12-token prefix into private pages of each branch (3 pages of 4)
    ps, H_kv, d = w.page_size, w.num_kv_heads, w.head_dim
    rows, pool_k, pool_v = [], [], []
    for b in range(2):
        ks, vs = context_by_walk(inp, b, ps)
        C = len(ks)
        npg = -(-C // ps)
        pk = torch.zeros(npg, H_kv, ps, d, dtype=inp.k_pages.dtype)
        pv = torch.zeros(npg, H_kv, ps, d, dtype=inp.v_pages.dtype)
        for i in range(C):
            pk[i // ps, :, i % ps] = torch.tensor(ks[i], dtype=inp.k_pages.dtype)
            pv[i // ps, :, i % ps] = torch.tensor(vs[i], dtype=inp.v_pages.dtype)
        base = sum(p.shape[0] for p in pool_k)
        rows.append(list(range(base, base + npg)))
        pool_k.append(pk)
        pool_v.append(pv)
    width = max(len(r) for r in rows)
    table3 = torch.tensor([r + [-1] * (width - len(r)) for r in rows], dtype=torch.int32)
    inp3 = Inputs(inp.q, inp.k_shared[:, :0], inp.v_shared[:, :0], torch.cat(pool_k),
                  torch.cat(pool_v), table3, [0], [0], [0, 0], inp.branch_q_len,
                  [12 + L for L in inp.branch_private_len])
    o3, l3 = run_oracle(w, inp3)
    assert torch.equal(o3, o) and torch.equal(l3, lse)


def pin_golden_append_placement():
    """Appended rows land where the paging rule puts them, worked by hand:
    4-token pages; branch 0 holds 3 private tokens in pages [5, 2, 7] and
    gets 4 more, so they fill slot 3 of page 5 and slots 0..2 of page 2;
    branch 1 holds none in pages [1, 6] and gets 2, slots 0 and 1 of page 1.
    Nothing else in the pool changes."""
    ps, n_pages = 4, 8
    k_pages = torch.arange(n_pages * 1 * ps * 2, dtype=torch.float32).view(n_pages, 1, ps, 2) * -1.0
    v_pages = k_pages - 1000.0
    table = torch.tensor([[5, 2, 7], [1, 6, -1]], dtype=torch.int32)
    k_new = torch.tensor([[[10.0, 11.0]], [[20.0, 21.0]], [[30.0, 31.0]], [[40.0, 41.0]],
                          [[50.0, 51.0]], [[60.0, 61.0]]])
    v_new = k_new + 0.5
    kp, vp = oracle.append_kv(k_pages, v_pages, table, [3, 0], [4, 2], k_new, v_new, ps)
    expected = {(5, 3): 0, (2, 0): 1, (2, 1): 2, (2, 2): 3, (1, 0): 4, (1, 1): 5}
    for page in range(n_pages):
        for slot in range(ps):
            if (page, slot) in expected:
                r = expected[(page, slot)]
                assert torch.equal(kp[page, :, slot], k_new[r]) and torch.equal(vp[page, :, slot], v_new[r])
            else:
                assert torch.equal(kp[page, :, slot], k_pages[page, :, slot])
                assert torch.equal(vp[page, :, slot], v_pages[page, :, slot])


def pin_invariant_append_then_attend():
    """Attention after appending a branch's last rows to a pool that lacked
    them equals attention over the pool that held them from the start."""
    w = custom("append", H_q=4, H_kv=2, d=16, page_size=4, shared=(10,),
               branches=((0, 3, 11), (0, 2, 6)), seed=31)
    inp = generate(w, "cpu")
    o, lse = run_oracle(w, inp)
    n_new = [5, 2]
    keep = [L - n for L, n in zip(inp.branch_private_len, n_new)]
    ks, vs, kp, vp = [], [], inp.k_pages.clone(), inp.v_pages.clone()
    for b, (k0, n) in enumerate(zip(keep, n_new)):
        walk_k, walk_v = context_by_walk(inp, b, w.page_size)
        C = len(walk_k)
        for i in range(n):
            ks.append(torch.tensor(walk_k[C - n + i], dtype=inp.k_pages.dtype))
            vs.append(torch.tensor(walk_v[C - n + i], dtype=inp.v_pages.dtype))
            page = int(inp.page_table[b][(k0 + i) // w.page_size])
            kp[page, :, (k0 + i) % w.page_size] = 0
            vp[page, :, (k0 + i) % w.page_size] = 0
    kp, vp = oracle.append_kv(kp, vp, inp.page_table, keep, n_new, torch.stack(ks), torch.stack(vs), w.page_size)
    inp2 = Inputs(inp.q, inp.k_shared, inp.v_shared, kp, vp, inp.page_table, inp.group_shared_start,
                  inp.group_shared_len, inp.branch_group, inp.branch_q_len, inp.branch_private_len)
    o2, l2 = run_oracle(w, inp2)
    assert torch.equal(o2, o) and torch.equal(l2, lse)


def pin_sampled_mode_equals_full_call():
    """A sampled call -- any subset of query tokens across branches and
    groups, any subset of query heads, in any order -- returns exactly the
    matching entries of the full call, bit for bit. Batching and sampling
    change only which rows are computed, never their value (ADR-0060 GQA
    fused attention, Algorithm lineage: no new mathematics; AHBM Agentic
    Runtime Architecture, §1.3: combined rows stay independent). Every
    full-size GPU parity test relies on this mode."""
    cases = [
        custom("sample_fanout", H_q=8, H_kv=2, d=16, page_size=4, shared=(23,),
               branches=((0, 5, 9), (0, 3, 14), (0, 6, 2)), seed=37),
        # two groups (an empty one holding independent requests) and a
        # zero-query branch between them
        custom("sample_groups", H_q=6, H_kv=3, d=8, page_size=3, shared=(0, 19),
               branches=((0, 1, 11), (0, 1, 4), (1, 0, 5), (1, 4, 7), (1, 2, 3)), seed=41),
        get_workload("tiny_fp32_fanout"),
    ]
    for w in cases:
        inp = generate(w, "cpu")
        o, lse = run_oracle(w, inp)
        n, H = o.shape[0], o.shape[1]
        rng = random.Random(w.seed)
        samples = [
            (list(range(n))[::-1], None),                       # every token, reversed
            (rng.sample(range(n), max(1, n // 2)), None),        # a shuffled subset across branches
            (None, list(range(H))[::-1]),                       # every head, reversed
            (rng.sample(range(n), max(1, n // 3)), rng.sample(range(H), max(1, H // 2))),
            ([n - 1], [0]),                                     # one entry
            ([0, n - 1], [H - 1, 0]),
        ]
        for toks, heads in samples:
            o2, l2 = run_oracle(w, inp, tokens=toks, heads=heads)
            ti = torch.tensor(list(range(n)) if toks is None else toks, dtype=torch.int64)
            hi = torch.tensor(list(range(H)) if heads is None else heads, dtype=torch.int64)
            assert torch.equal(o2, o[ti][:, hi]), (w.name, toks, heads)
            assert torch.equal(l2, lse[ti][:, hi]), (w.name, toks, heads)


ALL_PINS = [
    pin_golden_weights_123, pin_golden_paged_causal, pin_golden_merge,
    pin_brute_force_tiny, pin_library_sdpa, pin_closed_form_zero_q,
    pin_closed_form_prefill_row0, pin_closed_form_dominant_key,
    pin_invariant_batching, pin_invariant_split_merge, pin_invariant_causal,
    pin_invariant_gqa_map, pin_invariant_paging, pin_golden_append_placement,
    pin_invariant_append_then_attend, pin_sampled_mode_equals_full_call,
]


def failing_pins():
    """Names of the pins that fail on the oracle as currently bound."""
    bad = []
    for p in ALL_PINS:
        try:
            p()
        except Exception:          # an assertion, or a crash caused by the mistake
            bad.append(p.__name__)
    return bad
