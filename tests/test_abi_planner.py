"""Host-side checks: the C-ABI library loads and exports every declared
symbol, the planner partitions the visible (row, key) pairs exactly, honours
split overrides, drops causally dead work and rejects bad arguments. No GPU
is used (the planner entry point never touches a device)."""

import os
import re

import pytest

import gqa_attention_agentic_amd as G
from gqa_attention_agentic_amd import _lib
from workload import custom, get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _plan(w, splits="workload"):
    return G.plan_host(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.group_shared_start(),
                       [g.shared_len for g in w.groups], [b.group for b in w.branches],
                       [b.q_len for b in w.branches], [b.private_len for b in w.branches], w.causal,
                       splits=w.splits if splits == "workload" else splits, dtype=w.dtype)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    header = open(os.path.join(ROOT, "include", "gqa_attn.h")).read()
    declared = set(re.findall(r"\b(gqa_attn_\w+)\s*\(", header))
    assert declared == set(_lib.EXPORTED), declared ^ set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    probes = open(os.path.join(ROOT, "include", "gqa_probe.h")).read()
    declared = set(re.findall(r"\b(gqa_probe_\w+)\s*\(", probes))
    assert declared == set(_lib.PROBES), declared ^ set(_lib.PROBES)
    for name in declared:
        assert hasattr(lib, name), name


def _expected_pairs(w):
    """Visible (unit_slot, token, g, kv, unit-local key) pairs, from first
    principles: each group's prefix unit and each branch's suffix unit."""
    G_ = w.group_size
    ng = len(w.groups)
    pairs = set()
    qb = 0
    for bi, b in enumerate(w.branches):
        sl = w.groups[b.group].shared_len
        C = sl + b.private_len
        for t in range(b.q_len):
            p = C - b.q_len + t
            tok = qb + t
            for j in range(C):
                if w.causal and j > p:
                    continue
                slot, kl = (b.group, j) if j < sl else (ng + bi, j - sl)
                for g in range(G_):
                    for kv in range(w.num_kv_heads):
                        pairs.add((slot, tok, g, kv, kl))
        qb += b.q_len
    return pairs


def _covered_pairs(w, items):
    G_ = w.group_size
    ng = len(w.groups)
    qb = [0]
    for b in w.branches:
        qb.append(qb[-1] + b.q_len)
    # token range of each unit slot
    first_tok = {}
    for bi, b in enumerate(w.branches):
        first_tok.setdefault(b.group, qb[bi])
        first_tok[ng + bi] = qb[bi]
    got = []
    for (slot, kv, r0, nr, k0, k1, split, kern, _bin, _chain) in items:
        for r in range(r0, r0 + nr):
            tok = first_tok[slot] + r // G_
            g = r % G_
            # the planner only clamps whole tiles; per-row causality is masked in the kernel
            if slot < ng:
                bi = max(i for i in range(len(w.branches)) if qb[i] <= tok and w.branches[i].group == slot)
                key_pos0 = 0
            else:
                bi = slot - ng
                key_pos0 = w.groups[w.branches[bi].group].shared_len
            b = w.branches[bi]
            C = w.groups[b.group].shared_len + b.private_len
            p = C - b.q_len + (tok - qb[bi])
            for kl in range(k0, k1):
                if w.causal and key_pos0 + kl > p:
                    continue
                got.append((slot, tok, g, kv, kl))
    return got


CASES = [
    get_workload("tiny_fp32_fanout"),
    custom("fan", H_q=8, H_kv=2, shared=(300,), branches=((0, 5, 37), (0, 7, 50), (0, 20, 100)), seed=1),
    custom("pref", H_q=4, H_kv=1, shared=(700,), branches=((0, 700, 0),), seed=1, splits=[3, 0]),
    custom("mixed", H_q=8, H_kv=2, shared=(0, 130), seed=1,
           branches=((0, 1, 1), (0, 1, 70), (0, 1, 300), (1, 3, 40), (1, 2, 9))),
    custom("reach", H_q=4, H_kv=2, shared=(100,), branches=((0, 30, 10),), seed=1),
    custom("noncausal", H_q=4, H_kv=2, shared=(257,), branches=((0, 2, 3),), causal=False, seed=1,
           splits=[5, 2]),
    custom("join", H_q=8, H_kv=2, shared=(500,), branches=((0, 70, 70),), seed=1),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_items_partition_visible_pairs(w):
    items, splits, stats = _plan(w)
    got = _covered_pairs(w, items)
    assert len(got) == len(set(got)), "a visible pair is covered twice"
    assert set(got) == _expected_pairs(w)
    assert stats["n_items_wide"] + stats["n_items_narrow"] == len(items)
    # A unit on the 32-row kernel fits one M-tile, so a narrow item's tokens
    # hold at most 32 rows (the size of that kernel's combination table).
    for (_slot, _kv, r0, nr, _k0, _k1, _split, kern, _bin, _chain) in items:
        if kern == 1:
            assert r0 == 0 and nr <= 32


def test_split_override_honoured():
    w = CASES[1]
    for sp in ([1, 1, 1, 1], [4, 2, 3, 1], [9, 1, 5, 2]):
        items, splits, _ = _plan(w, splits=sp)
        assert splits == sp
        for slot in range(4):
            used = {it[6] for it in items if it[0] == slot}
            assert used == set(range(sp[slot])), (slot, used)


def test_pinned_split_counts():
    assert _plan(get_workload("tiny_fp32_fanout"))[1] == [3, 1, 1]
    assert _plan(get_workload("decode_8k"))[1] == [32, 0]
    assert _plan(get_workload("prefill_32k"))[1] == [8, 0]


@pytest.mark.parametrize("dtype,rows", [("bf16", 256), ("fp32", 128)])
def test_causal_skip_counts_lower_triangle(dtype, rows):
    """Prefill: processed KV tiles equal the lower-triangular tile count (per
    M-tile of rows / G tokens x G heads, 64-key tiles, shards of 4096); the
    bf16 MFMA kernel uses 256-row M-tiles, the fp32 one 128-row M-tiles."""
    w = custom("tri", H_q=64, H_kv=8, shared=(32768,), branches=((0, 32768, 0),), seed=1, splits=[8, 0],
               dtype=dtype)
    items, _, stats = _plan(w)
    tok = rows // 8
    expect, n_items = 0, 0
    for i in range(32768 // tok):
        kend = tok * i + tok                   # keys visible to the tile's last row
        for s in range(8):
            k0, k1 = 4096 * s, min(4096 * (s + 1), kend)
            if k0 < kend:
                expect += -(-(k1 - k0) // 64)
                n_items += 8
    assert stats["n_kv_tiles"] == expect * 8
    assert len(items) == n_items
    # without the causal clamp the grid would be (M-tiles) * 8 shards * 8 heads * 64 tiles
    assert stats["n_kv_tiles"] < (32768 // tok) * 8 * 8 * 64 * 0.52


def test_heuristic_fills_the_device():
    items, splits, _ = _plan(get_workload("fanout_8x20_32k"))
    wide = [it for it in items if it[7] == 0]
    assert 256 <= len(wide) <= 1024, len(wide)
    items, splits, _ = _plan(get_workload("mixed_32dec_64x4"))
    assert all(s >= 1 for s in splits[1:])


@pytest.mark.parametrize("n,L,items", [(1, 2048, 64), (1, 4096, 128), (1, 8192, 128), (1, 12288, 192),
                                        (1, 16384, 256), (1, 65536, 256), (4, 8192, 256), (16, 2048, 256),
                                        (2, 4096, 128)])
def test_decode_heuristic_items(n, L, items):
    """Decode-like units (<= 32 rows) are cut into equal shards of at least
    256 keys, about one item per 256 KiB of K/V, but no fewer than half and
    no more than one per resident workgroup (256 on the host planner's 256
    CUs), and each item gets a workgroup of its own."""
    from workload.configs import Branch, Group, _llama

    w = _llama("d", [Group(0)], [Branch(0, 1, L) for _ in range(n)], causal=True, seed=2)
    plan_items, splits, stats = _plan(w, splits=None)
    narrow = [it for it in plan_items if it[7] == 1]
    assert stats["n_items_wide"] == 0
    assert len(narrow) == items, (len(narrow), splits)
    assert len(set(splits[1:])) == 1
    assert all(it[5] - it[4] >= 256 or it[5] == L for it in narrow)
    assert max(it[8] for it in narrow) + 1 == len(narrow)      # one item per workgroup


def _item_cost(it):
    return it[5] - it[4] + 96       # keys plus the planner's fixed per-item cost


def _jobs(its):
    """Consecutive items of one workgroup grouped into jobs: an item on its
    own, or a chain (first item hands its state on, the rest continue)."""
    jobs = []
    for it in its:
        if jobs and it[9] & 1:
            jobs[-1].append(it)
        else:
            jobs.append([it])
    return jobs


def _job_cost(job):
    return sum(it[5] - it[4] for it in job) + 96 + 16 * (len(job) - 1)


@pytest.mark.parametrize("name", ["fanout_8x20_32k", "decode_8k", "prefill_32k", "mixed_32dec_64x4"])
def test_bins_pack_items_onto_resident_workgroups(name):
    """Each kernel's items are dealt to at most 256 workgroups (one per CU);
    a workgroup's items are contiguous and its jobs (items, or chains of
    one M-tile's shards) largest first; no workgroup's load exceeds the
    list-scheduling bound (mean load + largest job) by more than the 2% that
    the XCD placement may cost."""
    items, _, _ = _plan(get_workload(name))
    for kern in (0, 1):
        its = [it for it in items if it[7] == kern]
        if not its:
            continue
        bins = [it[8] for it in its]
        assert bins == sorted(bins), "items of a workgroup are not contiguous"
        n_bins = max(bins) + 1
        assert n_bins <= 256 and n_bins <= len(its)
        load = [0] * n_bins
        jobs = []
        for b in range(n_bins):
            jobs_b = _jobs([it for it in its if it[8] == b])
            costs = [_job_cost(j) for j in jobs_b]
            assert costs == sorted(costs, reverse=True), "jobs of a workgroup are not largest first"
            load[b] = sum(costs)
            jobs += jobs_b
        bound = sum(load) / n_bins + max(_job_cost(j) for j in jobs)
        assert max(load) <= 1.02 * bound, (max(load), bound)


def test_fanout_bins_balance_and_share_l2():
    """Fan-out: 240 prefix items (6 shards x 5 M-tiles x 8 KV heads) and 64
    suffix items fill exactly 256 workgroups, none holding two prefix items;
    the M-tiles of one (KV head, shard) sit on one XCD (bin residue mod 8)."""
    items, _, _ = _plan(get_workload("fanout_8x20_32k"))
    wide = [it for it in items if it[7] == 0]
    assert max(it[8] for it in wide) + 1 == 256
    per_bin = {}
    for it in wide:
        per_bin.setdefault(it[8], []).append(it)
    assert all(sum(1 for it in v if it[0] == 0) <= 1 for v in per_bin.values())
    xcd = {}
    for it in wide:
        xcd.setdefault((it[0], it[1], it[6]), set()).add(it[8] % 8)
    assert all(len(v) == 1 for v in xcd.values())


@pytest.mark.parametrize("name,rows,launch", [("decode_8k", True, 0), ("fanout_8x20_32k", True, 1),
                                              ("prefill_32k", False, 0), ("mixed_32dec_64x4", True, 1),
                                              ("join_8000_32k", False, 0)])
def test_merge_launch_only_when_wide_partials(name, rows, launch):
    """Rows whose partials all come from the narrow kernel are combined inside
    it: a decode forward has no separate merge launch; workloads with rows
    split over the MFMA kernel keep it. The prefill's 8 shards per M-tile
    form chains merged in registers: every row has one partial, written as
    the result, and nothing is left to merge."""
    _, _, stats = _plan(get_workload(name))
    assert (stats["n_merge_rows"] > 0) == rows
    assert stats["merge_launch"] == launch
    if not rows:
        assert stats["workspace_bytes"] == 0


def test_partials_packed_at_the_tile_rows():
    """A tile's partial rows are laid out at the tile's own row count: the 8k
    decode (one token, G = 8, 32 shards of 8 KV heads) needs 8 rows per
    (KV head, shard), not the 32-row kernel's full M-tile -- (m, l) as two
    floats then d fp32 values per row."""
    w = get_workload("decode_8k")
    _, _, stats = _plan(w)
    rows = w.num_kv_heads * 32 * w.group_size
    ml = -(-rows * 8 // 256) * 256
    assert stats["workspace_bytes"] == ml + rows * w.head_dim * 4


@pytest.mark.parametrize("name,chains", [("prefill_32k", True), ("join_8000_32k", True), ("fanout_8x20_32k", False),
                                         ("join_400_32k", False)])
def test_shards_of_an_m_tile_chain_when_work_is_plentiful(name, chains):
    """With at least two (unit, KV head, M-tile) jobs per workgroup the live
    shards of each job form a chain: consecutive items of one workgroup, in
    shard order over contiguous keys, the first handing its state on, the
    last writing it, those between doing both. A group with one branch
    chains the prefix's shards on into the suffix's (same KV head and rows),
    so the 8000-token join writes every row once. With fewer jobs (fan-out,
    400-token join) no item chains."""
    w = get_workload(name)
    items, splits, stats = _plan(w)
    wide = [it for it in items if it[7] == 0]
    chained = [it for it in wide if it[9]]
    if chains is False:
        assert not chained
        return
    assert chained
    if name == "join_8000_32k":
        assert stats["n_merge_rows"] == 0 and stats["workspace_bytes"] == 0
        assert all(it[9] for it in wide)
    for b in {it[8] for it in wide}:
        for job in _jobs([it for it in wide if it[8] == b]):
            if len(job) == 1:
                assert job[0][9] == 0
                continue
            assert len({(it[1], it[2], it[3]) for it in job}) == 1                 # one head, one M-tile
            units = [it[0] for it in job]
            assert units == sorted(units) and len(set(units)) <= 2
            if len(set(units)) == 2:                                               # prefix then suffix
                assert units[0] == 0 and units[-1] == 1 and len(w.branches) == 1
            for u in set(units):
                part = [it for it in job if it[0] == u]
                assert [it[6] for it in part] == list(range(len(part)))            # shard order
                assert all(a[5] == b[4] for a, b in zip(part, part[1:]))           # contiguous keys
            assert job[0][9] == 2 and job[-1][9] == 1 and all(it[9] == 3 for it in job[1:-1])


@pytest.mark.parametrize("name,split", [("decode_8k", False), ("fanout_8x20_32k", False),
                                        ("prefill_32k", False), ("mixed_32dec_64x4", True)])
def test_side_by_side_split(name, split):
    """A forward with items of both attention kernels gives each a disjoint
    share of the 256 CUs (a multiple of the 8 XCDs), and each kernel's items
    are dealt to at most that many workgroups; otherwise each kernel gets
    the whole device."""
    items, _, stats = _plan(get_workload(name))
    if split:
        assert stats["wide_cus"] + stats["narrow_cus"] == 256
        assert stats["wide_cus"] % 8 == 0 and 8 <= stats["narrow_cus"] <= 248
    else:
        assert stats["wide_cus"] == stats["narrow_cus"] == 256
    for kern, cus in ((0, stats["wide_cus"]), (1, stats["narrow_cus"])):
        bins = {it[8] for it in items if it[7] == kern}
        assert len(bins) <= cus and (not bins or max(bins) < cus)


BAD = [
    (dict(H_q=6, H_kv=4), "multiple"),
    (dict(d=96), "head_dim"),
    (dict(page_size=0), "page_size"),
]


@pytest.mark.parametrize("kw,msg", BAD)
def test_bad_params_rejected(kw, msg):
    args = dict(H_q=8, H_kv=2, d=128, page_size=16)
    args.update(kw)
    with pytest.raises(_lib.GqaError) as e:
        G.plan_host(args["H_q"], args["H_kv"], args["d"], args["page_size"], [0], [10], [0], [1], [0], True)
    assert msg in str(e.value)


@pytest.mark.parametrize("dtype,h_q,ok", [("bf16", 256, True), ("bf16", 512, False),
                                           ("fp32", 128, True), ("fp32", 256, False)])
def test_query_heads_per_kv_head_limit(dtype, h_q, ok):
    """An M-tile holds whole tokens, so one KV head serves at most as many
    query heads as the MFMA kernel has rows (256 bf16, 128 fp32); more is
    reported as unsupported."""
    def call():
        return G.plan_host(h_q, 1, 128, 16, [0], [500], [0], [3], [0], True, dtype=dtype)
    if ok:
        items, _, _ = call()
        assert items and all(r0 % h_q == 0 and nr % h_q == 0 for (_, _, r0, nr, *_rest) in items)
    else:
        with pytest.raises(_lib.GqaError) as e:
            call()
        assert e.value.status == -2 and "query heads per KV head" in str(e.value)


def test_m_tiles_hold_whole_tokens():
    """With G = 3 a 256-row tile would split a token; tiles hold 85 tokens
    (255 rows) instead, so every row of a token shares one M-tile."""
    w = custom("g3", H_q=6, H_kv=2, shared=(300,), branches=((0, 100, 50), (0, 90, 20)), seed=1)
    items, _, _ = _plan(w)
    assert items
    for (_slot, _kv, r0, nr, *_rest) in items:
        assert r0 % 3 == 0 and nr % 3 == 0 and nr <= 255
    assert set(_covered_pairs(w, items)) == _expected_pairs(w)


@pytest.mark.parametrize("agents,G", [(2, 8), (4, 8), (8, 8), (8, 2), (8, 4), (3, 1)])
def test_m_tiles_of_a_unit_are_balanced(agents, G):
    """A unit's work is spread evenly over its M-tiles in whole 32-row waves
    (active waves per tile differ by at most one, and no tile has a wave
    more than its rows need), so no tile of a shared prefix is a small
    remnant that streams the prefix's K/V at another pace than the others.
    (Coverage of these plans is checked on smaller prefixes above and in the
    sanitizer build.)"""
    w = custom("bal", H_q=8 * G, H_kv=8, shared=(32768,), branches=tuple((0, 20, 512) for _ in range(agents)),
               seed=3)
    items, _, _ = _plan(w)
    rows = {}
    for (slot, kv, r0, nr, *_rest) in items:
        rows.setdefault((slot, kv), set()).add((r0, nr))
    for key, tiles in rows.items():
        counts = [nr for _, nr in tiles]
        waves = [-(-nr // 32) for nr in counts]        # active 32-row waves of each tile
        assert max(waves) - min(waves) <= 1, (key, sorted(tiles))
        assert sum(waves) == -(-sum(counts) // 32), key   # no more waves than the rows need
        assert sum(counts) == (agents * 20 if key[0] == 0 else 20) * G, key


@pytest.mark.parametrize("meta,msg", [
    (([0], [10], [0], [12], [1]), "exceeds"),          # q_len > context
    (([0, 10], [10, 5], [0, 1, 0], [1, 1, 1], [0, 0, 0]), "consecutive"),
    (([0], [10], [0], [-1], [0]), "negative"),
    (([0], [10], [3], [1], [0]), "out of range"),
])
def test_bad_metadata_rejected(meta, msg):
    with pytest.raises(_lib.GqaError) as e:
        G.plan_host(8, 2, 128, 16, *meta, True)
    assert msg in str(e.value)


def test_bad_split_list_rejected():
    with pytest.raises(ValueError) as e:
        G.plan_host(8, 2, 128, 16, [0], [10], [0], [1], [0], True, splits=[1])
    assert "splits_override" in str(e.value)


class _StubLib:
    """Records the metadata arrays the binding hands to gqa_attn_forward."""

    def __init__(self):
        self.calls = []

    def gqa_attn_forward(self, *args):
        self.calls.append(args)
        return 0


def _stub_handle():
    h = object.__new__(G.GqaAttention)
    h.lib, h._h, h.dtype_code, h.num_q_heads = _StubLib(), None, _lib.GQA_BF16, 4
    h._meta_key = h._meta_arrays = None
    h._n_units = 0
    return h


def test_binding_reuses_metadata_arrays_and_sees_changes():
    """The binding converts the host metadata once per distinct value: a
    repeated call reuses the arrays, an in-place change of a list is seen,
    and wrong lengths are rejected before the library is called."""
    import torch
    h = _stub_handle()
    q = torch.zeros(3, 4, 8, dtype=torch.bfloat16)
    kv = torch.zeros(1, 16, 8, dtype=torch.bfloat16)
    pages = torch.zeros(2, 1, 4, 8, dtype=torch.bfloat16)
    table = torch.zeros(1, 2, dtype=torch.int32)
    gl, bq, bp = [16], [3], [5]
    args = (q, kv, kv, pages, pages, table, [0], gl, [0], bq, bp, True)
    h.forward(*args, stream=0)
    h.forward(*args, stream=0)
    a, b = h.lib.calls
    assert all(x is y for x, y in zip(a[10:16], b[10:16]))   # same ctypes arrays reused
    bp[0] = 6                                                # caller edits a list in place
    h.forward(*args, stream=0)
    c = h.lib.calls[-1]
    assert list(c[15])[:1] == [6]
    with pytest.raises(ValueError):
        h.forward(q, kv, kv, pages, pages, table, [0], gl, [0], bq, [5, 5], True, stream=0)
    with pytest.raises(ValueError):
        h.forward(q.float(), kv, kv, pages, pages, table, [0], gl, [0], bq, bp, True, stream=0)
    assert len(h.lib.calls) == 3
