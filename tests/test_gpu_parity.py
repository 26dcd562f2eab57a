"""HIP path against the fp64 oracle, element by element, on the GPU.

Small workloads (several KV tiles, ragged tails, every kernel instantiation,
paging with odd page sizes, causal edges) are compared on every output; the
full-size configurations are compared on sampled rows computed one by one by
the oracle. Tolerances: bf16 max-abs 2e-2 / mean-abs 2e-3 on O, fp32 1e-4;
LSE 1e-3 (bf16) / 1e-4 (fp32).
"""

import time

import pytest
import torch

from workload import custom, generate, get_workload
from workload.generate import Inputs

import gpu_helpers as H
import oracle

pytestmark = pytest.mark.gpu


SMALL = {
    "tiny_fp32_fanout": lambda: get_workload("tiny_fp32_fanout"),
    "fanout_bf16_d128": lambda: custom("fanout_bf16_d128", H_q=16, H_kv=2, d=128, page_size=16,
                                       shared=(1000,), branches=((0, 5, 37), (0, 7, 50), (0, 20, 100)),
                                       seed=101),
    "fanout_fp32_d128": lambda: custom("fanout_fp32_d128", dtype="fp32", H_q=16, H_kv=2, d=128,
                                       page_size=16, shared=(1000,),
                                       branches=((0, 5, 37), (0, 7, 50), (0, 20, 100)), seed=102),
    "fanout_bf16_d64_page12": lambda: custom("fanout_bf16_d64_page12", H_q=8, H_kv=2, d=64, page_size=12,
                                             shared=(333,), branches=((0, 9, 30), (0, 1, 0), (0, 4, 5)),
                                             seed=103),
    "fanout_fp32_d64_narrow": lambda: custom("fanout_fp32_d64_narrow", dtype="fp32", H_q=4, H_kv=2, d=64,
                                             page_size=8, shared=(150,), branches=((0, 2, 19), (0, 3, 7)),
                                             seed=104),
    "prefill_bf16": lambda: custom("prefill_bf16", shared=(700,), branches=((0, 700, 0),), seed=105,
                                   splits=[3, 0]),
    "prefill_fp32_d64": lambda: custom("prefill_fp32_d64", dtype="fp32", H_q=4, H_kv=1, d=64,
                                       shared=(300,), branches=((0, 300, 0),), seed=106),
    "decode_bf16": lambda: custom("decode_bf16", shared=(3000,), branches=((0, 1, 0),), causal=False,
                                  seed=107, splits=[8, 0]),
    "decode_bf16_d64": lambda: custom("decode_bf16_d64", d=64, shared=(2500,), branches=((0, 1, 0),),
                                      causal=False, seed=108),
    "mixed_bf16": lambda: custom("mixed_bf16", shared=(0, 500),
                                 branches=((0, 1, 1), (0, 1, 17), (0, 1, 300), (0, 1, 1000), (0, 1, 64))
                                 + tuple((1, 3, 40) for _ in range(6)), seed=109),
    "mha_g1": lambda: custom("mha_g1", H_q=4, H_kv=4, d=128, shared=(100,), branches=((0, 3, 20),),
                             seed=110),
    "gqa_g16": lambda: custom("gqa_g16", H_q=32, H_kv=2, d=128, shared=(200,),
                              branches=((0, 2, 10), (0, 3, 10)), seed=111),
    "gqa_g3_whole_token_tiles": lambda: custom("gqa_g3_whole_token_tiles", H_q=6, H_kv=2, d=128,
                                               shared=(300,), branches=((0, 100, 50), (0, 90, 20)),
                                               seed=117),
    "prefill_private_only": lambda: custom("prefill_private_only", shared=(0,), branches=((0, 50, 50),),
                                           seed=112),
    "queries_reach_into_prefix": lambda: custom("queries_reach_into_prefix", shared=(100,),
                                                branches=((0, 30, 10),), seed=113),
    "peaked_fanout": lambda: custom("peaked_fanout", shared=(1000,),
                                    branches=((0, 5, 37), (0, 7, 50), (0, 20, 100)), seed=114, q_scale=8.0),
    "zero_q_len_branch": lambda: custom("zero_q_len_branch", shared=(90,),
                                        branches=((0, 3, 10), (0, 0, 20), (0, 2, 5)), seed=115),
    "single_key": lambda: custom("single_key", shared=(1,), branches=((0, 1, 0),), seed=116),
    "join_continuation": lambda: custom("join_continuation", shared=(700,), branches=((0, 60, 60),),
                                        seed=118),
    # The largest query-head group one M-tile holds: 256 heads of one token
    # per KV head (bf16), 128 (fp32).
    "max_group_bf16": lambda: custom("max_group_bf16", H_q=256, H_kv=1, d=64, shared=(150,),
                                     branches=((0, 2, 30), (0, 3, 17)), seed=120),
    "max_group_fp32": lambda: custom("max_group_fp32", dtype="fp32", H_q=128, H_kv=1, d=64, page_size=8,
                                     shared=(90,), branches=((0, 2, 10),), seed=121),
    # Degenerate and large pages: one token per page, and a page far longer
    # than the suffix's tail.
    "page_size_1": lambda: custom("page_size_1", page_size=1, shared=(64,), branches=((0, 3, 9), (0, 2, 5)),
                                  seed=122),
    "page_size_512": lambda: custom("page_size_512", page_size=512, shared=(100,), branches=((0, 4, 700),),
                                    seed=123),
    # Forty one-token branches over one prefix: many tokens per narrow
    # M-tile, each combined inside the narrow launch.
    "many_branch_decode": lambda: custom("many_branch_decode", shared=(400,),
                                         branches=tuple((0, 1, k) for k in range(40)), seed=124),
    # Independent paged decodes of very different lengths (the split
    # heuristic gives each about one item per workgroup).
    "batched_paged_decodes": lambda: custom("batched_paged_decodes", shared=(0,),
                                            branches=((0, 1, 3000), (0, 1, 1200), (0, 1, 5000), (0, 1, 17)),
                                            seed=125),
    # 48 paged decodes forced to 4 shards each: 384 narrow items on at most
    # 256 workgroups, so workgroups run several items and the narrow kernel
    # takes its path for staggered arrivals (ordinary partial stores and a
    # release fence); the decodes above run one item per workgroup.
    "decodes_several_items_per_workgroup": lambda: custom(
        "decodes_several_items_per_workgroup", shared=(0,), branches=tuple((0, 1, 1500 + 37 * k) for k in range(48)),
        seed=127, splits=[0] + [4] * 48),
    # Long paged items in the narrow kernel (few shards, a dozen or more
    # tiles per wave), so each wave's next page ids are read a tile ahead,
    # over pages of 32 and 64 tokens with ragged last pages.
    "paged_decode_long_items_page32": lambda: custom("paged_decode_long_items_page32", page_size=32, shared=(0,),
                                                     branches=((0, 1, 6001),), seed=141, splits=[0, 2]),
    "paged_decode_long_items_d64_page64": lambda: custom("paged_decode_long_items_d64_page64", d=64, page_size=64,
                                                         shared=(0,), branches=((0, 1, 4099), (0, 1, 2500)),
                                                         seed=143, splits=[0, 1, 1]),
    # Decode-shaped tokens combined inside the narrow launch, past the fold's
    # first 64 partials (d = 128: one row per wave; d = 64: two rows per
    # wave), and with partials from both a prefix and a suffix unit.
    "decode_bf16_100_shards": lambda: custom("decode_bf16_100_shards", shared=(12800,), branches=((0, 1, 0),),
                                             causal=False, seed=133, splits=[100, 0]),
    "decode_bf16_d64_70_shards": lambda: custom("decode_bf16_d64_70_shards", d=64, shared=(7000,),
                                                branches=((0, 1, 0),), causal=False, seed=134, splits=[70, 0]),
    "decode_two_units_d128": lambda: custom("decode_two_units_d128", shared=(2000,), branches=((0, 1, 300),),
                                            seed=135, splits=[5, 3]),
    "decode_two_units_d64": lambda: custom("decode_two_units_d64", d=64, shared=(1500,), branches=((0, 1, 400),),
                                           seed=136, splits=[4, 6]),
    # Non-causal multi-token queries: every key of the context is visible.
    "noncausal_fanout": lambda: custom("noncausal_fanout", shared=(300,), branches=((0, 5, 40), (0, 7, 21)),
                                       causal=False, seed=126),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(name):
    H.full_parity(SMALL[name]())


def _random_workload(seed):
    """A seeded random configuration small enough for the oracle: 1-2
    groups, 1-4 branches each, any G, d, page size and causality, and the
    split counts either the heuristic's or random. Every branch's new tokens
    are at most its context."""
    import random
    r = random.Random(seed)
    dtype = "fp32" if r.random() < 0.2 else "bf16"
    H_kv = r.choice([1, 2, 4])
    G = r.choice([1, 2, 3, 4, 8])
    d = r.choice([64, 128])
    ps = r.choice([1, 4, 8, 12, 16, 32])
    n_groups = r.choice([1, 1, 2])
    shared = tuple(r.choice([0, r.randint(1, 700)]) for _ in range(n_groups))
    branches = []
    for g in range(n_groups):
        for _ in range(r.randint(1, 4)):
            priv = r.choice([0, r.randint(1, 300)])
            ctx = shared[g] + priv
            if ctx == 0:
                priv, ctx = 5, shared[g] + 5
            branches.append((g, r.randint(0, min(40, ctx)), priv))
    splits = None
    if r.random() < 0.5:
        splits = [r.randint(1, 9) for _ in range(n_groups + len(branches))]
    return custom(f"random_{seed}", dtype=dtype, H_q=H_kv * G, H_kv=H_kv, d=d, page_size=ps, shared=shared,
                  branches=tuple(branches), causal=r.random() < 0.8, seed=1000 + seed, splits=splits)


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations(seed):
    """Seeded random shapes across the planner's and kernels' paths (both
    attention kernels, paged and shared sources, ragged tiles, empty
    branches, forced and heuristic shards), every output against the
    oracle."""
    w = _random_workload(seed)
    H.say(f"  {w.name}: {w.dtype} H_q {w.num_q_heads} H_kv {w.num_kv_heads} d {w.head_dim} ps {w.page_size} "
          f"groups {[g.shared_len for g in w.groups]} branches {[(b.group, b.q_len, b.private_len) for b in w.branches]} "
          f"causal {w.causal} splits {w.splits}")
    if sum(b.q_len for b in w.branches) == 0:
        pytest.skip("no query tokens drawn")
    H.full_parity(w)


def _random_decode_workload(seed):
    """A seeded random decode-class configuration: many branches of one to
    four new tokens over shared and paged contexts, any G (odd ones too, so
    that a wave's rows belong to different tokens), d 64 or 128, and shard
    counts up to 40 -- the tokens whose partials all come from the 32-row
    kernel are combined inside its launch by the last item to finish."""
    import random
    r = random.Random(seed)
    dtype = "fp32" if r.random() < 0.2 else "bf16"
    H_kv = r.choice([1, 2, 4, 8])
    G = r.choice([1, 2, 3, 5, 8])
    d = r.choice([64, 128])
    ps = r.choice([1, 8, 16])
    n_groups = r.choice([1, 2])
    shared = tuple(r.choice([0, r.randint(100, 3000)]) for _ in range(n_groups))
    branches = []
    for g in range(n_groups):
        for _ in range(r.randint(1, 6)):
            priv = r.choice([0, r.randint(1, 2000)])
            if shared[g] + priv == 0:
                priv = r.randint(1, 500)
            branches.append((g, min(r.choice([1, 1, 1, 2, 4]), shared[g] + priv), priv))
    splits = None
    if r.random() < 0.7:
        splits = [r.randint(1, 40) for _ in range(n_groups + len(branches))]
    return custom(f"random_decode_{seed}", dtype=dtype, H_q=H_kv * G, H_kv=H_kv, d=d, page_size=ps,
                  shared=shared, branches=tuple(branches), causal=r.random() < 0.5, seed=2000 + seed,
                  splits=splits)


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_configurations(seed):
    """Seeded random decode-class shapes (the in-launch combination with
    partial counts up to 40 per unit, from one or two units, rows of several
    tokens per item), every output against the oracle."""
    w = _random_decode_workload(seed)
    H.say(f"  {w.name}: {w.dtype} H_q {w.num_q_heads} H_kv {w.num_kv_heads} d {w.head_dim} ps {w.page_size} "
          f"groups {[g.shared_len for g in w.groups]} branches {[(b.group, b.q_len, b.private_len) for b in w.branches]} "
          f"causal {w.causal} splits {w.splits}")
    H.full_parity(w)


@pytest.mark.parametrize("splits", [[4, 2, 1, 3], [1, 1, 1, 1], [16, 5, 4, 9]])
def test_split_override(splits):
    w = SMALL["fanout_bf16_d128"]()
    H.full_parity(w, splits=splits, label=f"splits={splits}")


def test_empty_forward():
    w = custom("empty", shared=(10,), branches=((0, 0, 5),), seed=117)
    inp = generate(w, "cuda")
    h = H.handle_for(w)
    o, lse = h.forward_inputs(inp, True)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and lse.shape[0] == 0


def test_invariant_batching_on_gpu():
    """Fan-out computed together equals each branch computed alone."""
    w = SMALL["fanout_bf16_d128"]()
    inp = generate(w, "cuda")
    o, lse, _ = H.run_library(w, inp)
    qb = 0
    for b in range(len(w.branches)):
        T = inp.branch_q_len[b]
        alone = Inputs(inp.q[qb:qb + T].contiguous(), inp.k_shared, inp.v_shared, inp.k_pages,
                       inp.v_pages, inp.page_table[b:b + 1].contiguous(), inp.group_shared_start,
                       inp.group_shared_len, [0], [T], [inp.branch_private_len[b]])
        o1, l1, _ = H.run_library(w, alone, splits=None)
        assert (o1.float() - o[qb:qb + T].float()).abs().max().item() < 2e-2
        assert (l1 - lse[qb:qb + T]).abs().max().item() < 1e-3
        qb += T


def test_invariant_splits_on_gpu():
    """One shard (direct O / l write) and many shards (merge) agree."""
    w = SMALL["fanout_bf16_d128"]()
    inp = generate(w, "cuda")
    o1, l1, _ = H.run_library(w, inp, splits=[1, 1, 1, 1])
    o2, l2, h2 = H.run_library(w, inp, splits=[13, 3, 2, 4])
    assert h2.plan_stats()["n_merge_rows"] > 0
    assert (o1.float() - o2.float()).abs().max().item() < 2e-2
    assert (l1 - l2).abs().max().item() < 1e-3


def test_invariant_page_permutation_bitwise():
    """Renumbering physical pages (table rewritten) leaves the result
    bit-identical: pages are referenced, never copied."""
    w = SMALL["fanout_bf16_d128"]()
    inp = generate(w, "cuda")
    o1, l1, _ = H.run_library(w, inp)
    n = inp.k_pages.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).to("cuda")
    kp = torch.empty_like(inp.k_pages)
    vp = torch.empty_like(inp.v_pages)
    kp[perm] = inp.k_pages
    vp[perm] = inp.v_pages
    table = inp.page_table.clone()
    valid = table >= 0
    table[valid] = perm[table[valid].long()].int()
    inp2 = Inputs(inp.q, inp.k_shared, inp.v_shared, kp, vp, table, inp.group_shared_start,
                  inp.group_shared_len, inp.branch_group, inp.branch_q_len, inp.branch_private_len)
    o2, l2, _ = H.run_library(w, inp2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_determinism_bitwise():
    w = SMALL["mixed_bf16"]()
    inp = generate(w, "cuda")
    h = H.handle_for(w)
    o1, l1, _ = H.run_library(w, inp, handle=h)
    o1, l1 = o1.clone(), l1.clone()
    for _ in range(3):
        o2, l2, _ = H.run_library(w, inp, handle=h)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_alternating_plans_on_one_handle():
    """One handle alternating between two plans (fan-out with a split prefix,
    then a 6-shard decode) four times: the per-token arrival counters of the
    in-launch combination must be back at zero after every forward, and be
    cleared when the layout changes, so every result matches the oracle and
    repeats bit for bit."""
    wa = custom("alt_fanout", H_q=16, H_kv=2, d=128, page_size=16, shared=(900,),
                branches=((0, 5, 37), (0, 7, 50), (0, 3, 9)), seed=121, splits=[4, 1, 1, 1])
    wb = custom("alt_decode", H_q=16, H_kv=2, d=128, shared=(1500,), branches=((0, 1, 0),), causal=False,
                seed=122, splits=[6, 0])
    ia, ib = generate(wa, "cuda"), generate(wb, "cuda")
    ra, rb = H.oracle_rows(wa, ia), H.oracle_rows(wb, ib)
    h = H.handle_for(wa)
    first = {}
    for rep in range(4):
        for w, inp, ref in ((wa, ia, ra), (wb, ib, rb)):
            o, lse, _ = H.run_library(w, inp, handle=h)
            H.compare(w, o, lse, ref[0], ref[1], ref[2], label=f"{w.name} #{rep}")
            if w.name in first:
                assert torch.equal(o, first[w.name][0]) and torch.equal(lse, first[w.name][1]), w.name
            else:
                first[w.name] = (o.clone(), lse.clone())


def test_side_by_side_kernels_join_the_callers_stream():
    """A forward with items of both attention kernels runs them side by side
    (the narrow one on the handle's side stream) on a split of the CUs. The
    caller's stream must still see the finished result: copies queued right
    after the forward on the same non-default stream match the oracle, and
    the kernel timing reports one forward."""
    w = SMALL["mixed_bf16"]()
    inp = generate(w, "cuda")
    ref = H.oracle_rows(w, inp)
    h = H.handle_for(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    h.enable_timing(True)
    with torch.cuda.stream(s):
        o, lse = h.forward_inputs(inp, w.causal, splits=w.splits, stream=s.cuda_stream)
        o_copy, lse_copy = o.clone(), lse.clone()
    s.synchronize()
    stats = h.plan_stats()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert stats["wide_cus"] + stats["narrow_cus"] == n_cu and 0 < stats["narrow_cus"] < n_cu
    attn_ms, _, n = h.kernel_times()
    assert n == 1 and attn_ms > 0
    H.compare(w, o_copy, lse_copy, ref[0], ref[1], ref[2], label="side by side")


def test_keys_past_the_prefix_extent_ignored():
    """NaN keys and values stored after a group's prefix (past its extent in
    k_shared) are never read: the result is bit-identical."""
    w = custom("future", shared=(200,), branches=((0, 64, 0),), seed=118)
    inp = generate(w, "cuda")
    o1, l1, _ = H.run_library(w, inp)
    # positions of the queries are 136..199: poison nothing visible -> same
    # result; then poison a key no query sees by shrinking the context.
    w2 = custom("future2", shared=(200,), branches=((0, 64, 0),), seed=118)
    inp2 = generate(w2, "cuda")
    k2 = torch.cat([inp2.k_shared, torch.full_like(inp2.k_shared[:, :8], float("nan"))], 1).contiguous()
    v2 = torch.cat([inp2.v_shared, torch.full_like(inp2.v_shared[:, :8], float("nan"))], 1).contiguous()
    inp3 = Inputs(inp2.q, k2, v2, inp2.k_pages, inp2.v_pages, inp2.page_table, [0], [200], [0], [64], [0])
    o3, l3, _ = H.run_library(w2, inp3)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_causal_future_key_inside_the_context_ignored():
    """A prefill of 200 tokens with key 150 poisoned (K NaN, V 1e4, every KV
    head): rows before position 150 never see it -- they stay finite and
    match the oracle -- while rows from 150 on do see it. Covers a causal
    diagonal inside one M-tile and one KV tile."""
    w = custom("future_inside", shared=(200,), branches=((0, 200, 0),), seed=119)
    inp = generate(w, "cuda")
    ref = H.oracle_rows(w, inp)
    j = 150
    inp.k_shared[:, j] = float("nan")
    inp.v_shared[:, j] = 1e4
    o, lse, _ = H.run_library(w, inp)
    H.compare(w, o, lse, ref[0][:j], ref[1][:j], list(range(j)), label="rows before the poisoned key")
    assert not torch.isfinite(o[j:].float()).all(), "rows that see the NaN key should not be finite"


@pytest.mark.parametrize("name", ["fanout_bf16_d128", "fanout_fp32_d128", "mixed_bf16", "page_size_512",
                                  "fanout_bf16_d64_page12"])
def test_unused_slots_of_last_pages_never_read(name):
    """NaN in every unused slot of each branch's last (partial) page, and in
    the spare pages of the pool: the result is bit-identical to the clean
    run, so no kernel reads past a suffix's end."""
    w = SMALL[name]()
    inp = generate(w, "cuda")
    o1, l1, _ = H.run_library(w, inp)
    o1, l1 = o1.clone(), l1.clone()
    ps = w.page_size
    used = set()
    kp, vp = inp.k_pages.clone(), inp.v_pages.clone()
    for b, L in enumerate(inp.branch_private_len):
        npg = -(-L // ps)
        for p in range(npg):
            used.add(int(inp.page_table[b, p]))
        if L % ps:
            last = int(inp.page_table[b, npg - 1])
            kp[last, :, L % ps:] = float("nan")
            vp[last, :, L % ps:] = float("nan")
    for p in range(kp.shape[0]):
        if p not in used:
            kp[p] = float("nan")
            vp[p] = float("nan")
    poisoned = Inputs(inp.q, inp.k_shared, inp.v_shared, kp, vp, inp.page_table, inp.group_shared_start,
                      inp.group_shared_len, inp.branch_group, inp.branch_q_len, inp.branch_private_len)
    o2, l2, _ = H.run_library(w, poisoned)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,d,n,splits", [("bf16", 128, 4096, 4), ("fp32", 64, 2048, 3)])
def test_chained_shards_prefill(dtype, d, n, splits):
    """A causal prefill with H_q 64, H_kv 8 and pinned shards, long enough
    that its (KV head, M-tile) jobs outnumber the workgroups twice over: the
    shards of each M-tile run as a chain, merged in registers, and every row
    is written directly (no partials, no merge launch). Compared with the
    oracle on every 8th token plus the M-tile, KV-tile and shard edges."""
    w = custom(f"chain_prefill_{dtype}", dtype=dtype, H_q=64, H_kv=8, d=d, shared=(n,), branches=((0, n, 0),),
               seed=131, splits=[splits, 0])
    inp = generate(w, "cuda")
    o, lse, h = H.run_library(w, inp)
    st = h.plan_stats()
    H.say(f"  {w.name}: plan {st}")
    assert st["merge_launch"] == 0 and st["n_merge_rows"] == 0 and st["workspace_bytes"] == 0
    m_tile = (256 if dtype == "bf16" else 128) // 8
    toks = sorted(set(range(0, n, 8)) | _edges(n, -(-n // splits), m_tile))
    ref = H.oracle_rows(w, inp, tokens=toks)
    H.compare(w, o, lse, ref[0], ref[1], ref[2], label=f"{w.name} ({len(toks)}/{n} tokens)")


@pytest.mark.parametrize("dtype,d,n_shared,n,splits", [("bf16", 128, 3000, 2048, [2, 2]),
                                                        ("fp32", 64, 1500, 1024, [1, 3])])
def test_chained_join_prefix_into_suffix(dtype, d, n_shared, n, splits):
    """A join: one branch of n new tokens over an n_shared-token prefix, with
    jobs enough to chain. Each (KV head, M-tile) chain runs the prefix's
    shards and then the suffix's, so the state crosses from the shared keys
    to the paged ones in registers and every row is written once (no
    partials, no merge launch). Compared with the oracle on every 8th token
    plus the M-tile and shard edges."""
    w = custom(f"chain_join_{dtype}", dtype=dtype, H_q=64, H_kv=8, d=d, shared=(n_shared,), branches=((0, n, n),),
               seed=132, splits=splits)
    inp = generate(w, "cuda")
    o, lse, h = H.run_library(w, inp)
    st = h.plan_stats()
    H.say(f"  {w.name}: plan {st}")
    assert st["merge_launch"] == 0 and st["n_merge_rows"] == 0 and st["workspace_bytes"] == 0
    m_tile = (256 if dtype == "bf16" else 128) // 8
    toks = sorted(set(range(0, n, 8)) | _edges(n, -(-n // splits[1]), m_tile))
    ref = H.oracle_rows(w, inp, tokens=toks)
    H.compare(w, o, lse, ref[0], ref[1], ref[2], label=f"{w.name} ({len(toks)}/{n} tokens)")


# ------------------------------------------------ full-size configurations --
def _parity(name, tokens=None):
    """The library's output at a full-size workload against the oracle on
    `tokens` (global ids; None: every token), all heads. Max-abs and mean-abs
    are taken over every compared element."""
    w = get_workload(name)
    H.say(f"[parity] {name}: generating")
    inp = generate(w, "cuda")
    H.say(f"[parity] {name}: library")
    o, lse, h = H.run_library(w, inp)
    H.say(f"[parity] {name}: plan {h.plan_stats()} splits {h.plan_splits()[:6]}")
    toks = list(range(w.n_q_tokens)) if tokens is None else list(tokens)
    n = len(toks)
    H.say(f"[parity] {name}: oracle on {n} of {w.n_q_tokens} tokens x {w.num_q_heads} heads")
    # The oracle in pieces of a branch (or 128 tokens) at a time, with a
    # progress line after each: a sampled oracle call returns exactly the
    # full call's entries, so the pieces concatenate to the full result.
    qb = [0]
    for b in w.branches:
        qb.append(qb[-1] + b.q_len)
    pieces, o_parts, l_parts, t0 = [], [], [], time.time()
    for b in range(len(w.branches)):
        mine = [t for t in toks if qb[b] <= t < qb[b + 1]]
        pieces += [(b, mine[i:i + 128]) for i in range(0, len(mine), 128)]
    for k, (b, part) in enumerate(pieces):
        o_p, l_p, _ = H.oracle_rows(w, inp, branches=[b], tokens=part)
        o_parts.append(o_p)
        l_parts.append(l_p)
        if k % 8 == 7 or k == len(pieces) - 1:
            H.say(f"[parity] {name}: oracle piece {k + 1}/{len(pieces)}, {time.time() - t0:.0f}s")
    order = [t for _, part in pieces for t in part]
    o_ref, l_ref = torch.cat(o_parts), torch.cat(l_parts)
    return H.compare(w, o, lse, o_ref, l_ref, order, label=f"{name} ({n}/{w.n_q_tokens} tokens)")


def test_tiny_fp32_fanout_full():
    H.full_parity(get_workload("tiny_fp32_fanout"))


def test_decode_8k_full():
    _parity("decode_8k")


def test_fanout_8x20_32k_all_160_tokens():
    _parity("fanout_8x20_32k")


def _edges(n, shard, m_tile, kv_tile=64):
    """Token ids next to shard, M-tile and KV-tile boundaries, and the ends."""
    out = {0, 1, n - 2, n - 1}
    for step in (shard, m_tile, kv_tile):
        for b in range(step, n, step):
            if step != kv_tile or b % 1024 == 0:   # KV-tile edges: a spread of them
                out |= {b - 1, b}
    return {t for t in out if 0 <= t < n}


@pytest.mark.timeout(900)
def test_prefill_32k_every_16th_token_and_edges():
    """1 token in 16 (2048 rows per head, every 32-token M-tile hit twice)
    plus the tokens on each side of the 8 shard boundaries, every M-tile
    boundary and a spread of KV-tile boundaries."""
    toks = set(range(0, 32768, 16)) | _edges(32768, 4096, 32)
    _parity("prefill_32k", sorted(toks))


@pytest.mark.timeout(900)
def test_mixed_32dec_64x4_all_288_tokens():
    _parity("mixed_32dec_64x4")


@pytest.mark.timeout(600)
def test_join_400_32k_all_400_tokens():
    """Continuation prefill after a join: the new tokens see the whole prefix
    and the join input up to themselves."""
    _parity("join_400_32k")


@pytest.mark.timeout(900)
def test_join_8000_32k_every_16th_token_and_edges():
    toks = set(range(0, 8000, 16)) | _edges(8000, 1000, 32)
    _parity("join_8000_32k", sorted(toks))


def _passes(w, o, lse, o_ref, l_ref, toks, label):
    try:
        H.compare(w, o, lse, o_ref, l_ref, toks, label=label)
        return True
    except AssertionError:
        return False


def test_parity_check_rejects_planted_mistakes():
    """Mutation sanity on peaked scores: the library's output passes against
    the oracle, and fails against the oracle run on CPU inputs with a planted
    mistake -- the first third of the shared prefix (a shard) dropped, the
    private suffixes skipped, or two pages of a branch swapped."""
    w = SMALL["peaked_fanout"]()
    inp = generate(w, "cuda")
    o, lse, _ = H.run_library(w, inp)
    sub, toks = H.cpu_subset(inp, range(len(inp.branch_q_len)))

    def ref(x):
        return oracle.attention(x, w.num_kv_heads, w.page_size, w.causal)

    o_ref, l_ref = ref(sub)
    assert _passes(w, o, lse, o_ref, l_ref, toks, "correct oracle")
    L = sub.group_shared_len[0]
    a = L // 3
    dropped = Inputs(sub.q, sub.k_shared[:, a:].contiguous(), sub.v_shared[:, a:].contiguous(), sub.k_pages,
                     sub.v_pages, sub.page_table, [0], [L - a], sub.branch_group, sub.branch_q_len,
                     sub.branch_private_len)
    no_suffix = Inputs(sub.q, sub.k_shared, sub.v_shared, sub.k_pages, sub.v_pages, sub.page_table,
                       sub.group_shared_start, sub.group_shared_len, sub.branch_group, sub.branch_q_len,
                       [0] * len(sub.branch_private_len))
    table = sub.page_table.clone()
    table[0, 1], table[0, 2] = sub.page_table[0, 2], sub.page_table[0, 1]
    swapped = Inputs(sub.q, sub.k_shared, sub.v_shared, sub.k_pages, sub.v_pages, table,
                     sub.group_shared_start, sub.group_shared_len, sub.branch_group, sub.branch_q_len,
                     sub.branch_private_len)
    for label, x in (("shard dropped", dropped), ("suffix skipped", no_suffix), ("pages swapped", swapped)):
        o_bad, l_bad = ref(x)
        assert not _passes(w, o, lse, o_bad, l_bad, toks, label), f"planted mistake '{label}' passed"
