"""fp64 reference of shared-prefix GQA attention (test infrastructure only).

Sources (page titles; sections as they appear on the pages):

* AHBM Agentic Runtime Architecture, §3.1 -- a branch's page table is the
  shared prefix pages followed by its private pages; shared pages are
  referenced, never copied.
* same page, §1.3 and §3.2 -- combined-Q batching changes the execution
  shape only; every query row stays independent.
* ADR-0060 GQA fused attention, §3 (per-tile op sequence) -- scores are
  Q.K^T times softmax_scale, an additive mask removes invisible keys, then
  max / exp / sum / P.V.
* same page, §0.5.3 -- softmax_scale = 1/sqrt(d); the G query heads of one
  KV head form the query group.
* same page, §5.4 -- causal visibility of a key tile against a query block.
* same page, §4 -- the (m, l, O) merge: m = max(m_a, m_b), each side scaled
  by exp(m_side - m), the output normalised once at the end.

Readings where the pages leave a step open:

* query head h reads KV head floor(h / G) (contiguous groups);
* the q_len new tokens of a branch are the last q_len positions of its
  context; key j has position j;
* causal visibility is inclusive: key position <= query position;
* private token i of a branch is in page ``page_table[b][i // page_size]``
  at slot ``i % page_size``;
* a row that sees no key yields the merge identity (m, l, O) = (-inf, 0, 0);
  finalising it gives O = 0 and LSE = -inf;
* LSE = m + ln(l) in scaled-score units (natural log).
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import torch

F64 = torch.float64
EMPTY_LSE = float("-inf")


# ---------------------------------------------------------------- indexing --
def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: the G = H_q / H_kv query heads of one
    KV head are contiguous (ADR-0060 GQA fused attention, §0.5.3: Q group
    [G, T_q, d] per KV head)."""
    return h // (num_q_heads // num_kv_heads)


def default_scale(d: int) -> float:
    """softmax_scale = 1/sqrt(d) (ADR-0060 GQA fused attention, §0.5.3)."""
    return 1.0 / math.sqrt(d)


def lse_of(m: torch.Tensor, l: torch.Tensor) -> torch.Tensor:
    """Log-sum-exp of a row from its running max and sum: m + ln(l)."""
    return m + torch.log(l)


def query_positions(context_len: int, q_len: int) -> torch.Tensor:
    """Positions of a branch's new query tokens: the last q_len positions of
    its context (ADR-0060, §0.5.3 q_block_meta {q_start, T_q}; the new K/V
    are appended before launch, §0.5.1 precondition P3)."""
    return torch.arange(context_len - q_len, context_len, dtype=torch.int64)


def key_visible(key_pos: torch.Tensor, query_pos: torch.Tensor, causal: bool) -> torch.Tensor:
    """Boolean [n_query, n_key]: inclusive causal diagonal (ADR-0060, §5.4
    tile classes); without causality every key of the context is visible
    (§5.2: decode attends all past KV)."""
    if not causal:
        return torch.ones(query_pos.numel(), key_pos.numel(), dtype=torch.bool)
    return key_pos.view(1, -1) <= query_pos.view(-1, 1)


def private_location(i: int, page_size: int) -> Tuple[int, int]:
    """(logical page, slot) of private token i: tokens are appended to the
    branch's pages contiguously (AHBM Agentic Runtime Architecture, §3.1;
    ADR-0060, §2.1)."""
    return i // page_size, i % page_size


def append_kv(k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
              private_len: Sequence[int], n_new: Sequence[int], k_new: torch.Tensor, v_new: torch.Tensor,
              page_size: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """The page pools after appending new rows to each branch's private
    suffix (AHBM Agentic Runtime Architecture, §3.1: a branch's tokens go to
    its own pages, slot after slot; ADR-0060 GQA fused attention, §0.5.1: the
    cache is written before attention reads it). k_new / v_new hold branch
    b's n_new[b] rows ([rows, H_kv, d]) contiguously, branches in order; row
    i of branch b becomes private token private_len[b] + i. Returns CPU
    copies of the pools; the inputs are left as they are."""
    kp, vp = k_pages.to("cpu").clone(), v_pages.to("cpu").clone()
    kn, vn = k_new.to("cpu"), v_new.to("cpu")
    table = page_table.to("cpu").tolist()
    r = 0
    for b in range(len(n_new)):
        for i in range(n_new[b]):
            lp, slot = private_location(private_len[b] + i, page_size)
            page = table[b][lp]
            kp[page, :, slot, :] = kn[r]
            vp[page, :, slot, :] = vn[r]
            r += 1
    return kp, vp


# ----------------------------------------------------------------- context --
def branch_context(inp, b: int, page_size: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """K_b, V_b as float64 [C_b, H_kv, d]: the group's shared prefix followed
    by the branch's private suffix read through its page table
    (AHBM Agentic Runtime Architecture, §3.1 branch page table). The values
    are stored KV-head-major, so that ``K_b[:, kv]`` is contiguous."""
    g = inp.branch_group[b]
    s0, sl = inp.group_shared_start[g], inp.group_shared_len[g]
    n_priv = inp.branch_private_len[b]
    H_kv, d = inp.k_shared.shape[0], inp.k_shared.shape[2]
    out = []
    for src_shared, src_pages in ((inp.k_shared, inp.k_pages), (inp.v_shared, inp.v_pages)):
        ctx = torch.empty(H_kv, sl + n_priv, d, dtype=F64)
        ctx[:, :sl].copy_(src_shared[:, s0:s0 + sl, :])
        if n_priv > 0:
            table = inp.page_table[b].to("cpu").tolist()
            pages, slots = [], []
            for i in range(n_priv):
                lp, slot = private_location(i, page_size)
                pages.append(table[lp])
                slots.append(slot)
            pages_t = torch.tensor(pages, dtype=torch.int64, device=src_pages.device)
            slots_t = torch.tensor(slots, dtype=torch.int64, device=src_pages.device)
            priv = src_pages[pages_t, :, slots_t, :]              # [n_priv, H_kv, d]
            ctx[:, sl:].copy_(priv.permute(1, 0, 2))
        out.append(ctx.permute(1, 0, 2))                          # [C, H_kv, d] view
    return out[0], out[1]


def _branch_q_begin(inp) -> List[int]:
    out, acc = [], 0
    for t in inp.branch_q_len:
        out.append(acc)
        acc += t
    return out


# ---------------------------------------------------------- full attention --
def _softmax_rows(z: torch.Tensor, v: torch.Tensor):
    """Full softmax over the last axis of z [..., C] (invisible keys hold
    -inf) and its product with v [C, d]; returns (O, LSE). Rows with no
    visible key give O = 0, LSE = -inf."""
    m = z.max(dim=-1, keepdim=True).values
    empty = torch.isinf(m) & (m < 0)
    m_safe = torch.where(empty, torch.zeros_like(m), m)
    p = torch.exp(z - m_safe)                      # exp(-inf) = 0 for masked keys
    l = p.sum(dim=-1, keepdim=True)
    o = (p @ v) / torch.where(empty, torch.ones_like(l), l)
    lse = torch.where(empty, torch.full_like(m, EMPTY_LSE), lse_of(m, l))
    return o, lse.squeeze(-1)


def sample_slots(items: Sequence[int]) -> dict:
    """Output slot of each requested token (or head) id: its place in the
    list as the caller gave it (any order, any subset)."""
    return {x: i for i, x in enumerate(items)}


def heads_of_kv(kv: int, num_q_heads: int, num_kv_heads: int) -> List[int]:
    """The query heads that read KV head kv, through kv_head_of."""
    return [h for h in range(num_q_heads) if kv_head_of(h, num_q_heads, num_kv_heads) == kv]


def attention(inp, num_kv_heads: int, page_size: int, causal: bool,
              softmax_scale: Optional[float] = None,
              tokens: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[int]] = None):
    """O [n_tok, H_q, d] and LSE [n_tok, H_q] in float64.

    ``tokens`` (global query-token indices, any order, any branches) and
    ``heads`` restrict the computation to a sample; the returned tensors
    then have shape [len(tokens), len(heads), d] and [len(tokens),
    len(heads)], in the order given.

    Every value comes from the same computation whether it is requested
    alone or with all others: the unit of work is one query token against
    one KV head, i.e. the scores of that token's query heads of the KV head
    over the branch's whole context (one fixed-shape product with the KV
    head's keys, then one with its values). A sample therefore returns
    exactly the matching entries of the full call.
    """
    n_tok, H_q, d = inp.q.shape
    scale = default_scale(d) if softmax_scale is None else softmax_scale
    q_begin = _branch_q_begin(inp)
    tok_list = list(range(n_tok)) if tokens is None else list(tokens)
    head_list = list(range(H_q)) if heads is None else list(heads)
    out_o = torch.zeros(len(tok_list), len(head_list), d, dtype=F64)
    out_l = torch.full((len(tok_list), len(head_list)), EMPTY_LSE, dtype=F64)
    row_of = sample_slots(tok_list)
    col_of = sample_slots(head_list)
    kv_list = sorted({kv_head_of(h, H_q, num_kv_heads) for h in head_list})
    for b in range(len(inp.branch_q_len)):
        T = inp.branch_q_len[b]
        mine = [t for t in range(q_begin[b], q_begin[b] + T) if t in row_of]
        if not mine:
            continue
        kb, vb = branch_context(inp, b, page_size)
        C = kb.shape[0]
        qpos_all = query_positions(C, T)
        kpos = torch.arange(C, dtype=torch.int64)
        for kv in kv_list:
            k_kv = kb[:, kv, :].contiguous()             # [C, d]
            v_kv = vb[:, kv, :].contiguous()
            hs = heads_of_kv(kv, H_q, num_kv_heads)
            wanted = [(i, h) for i, h in enumerate(hs) if h in col_of]
            hsel = torch.tensor(hs, dtype=torch.int64, device=inp.q.device)
            for t in mine:
                q_blk = inp.q[t].index_select(0, hsel).to("cpu", F64).contiguous()   # [len(hs), d]
                vis = key_visible(kpos, qpos_all[t - q_begin[b]].view(1), causal)  # [1, C]
                z = scale * (q_blk @ k_kv.T)                                       # [len(hs), C]
                z = z.masked_fill(~vis, float("-inf"))
                o, lse = _softmax_rows(z, v_kv)
                for i, h in wanted:
                    out_o[row_of[t], col_of[h]] = o[i]
                    out_l[row_of[t], col_of[h]] = lse[i]
    return out_o, out_l


# ------------------------------------------------------ partials and merge --
def partial_state(q_rows: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  key_pos: torch.Tensor, row_pos: torch.Tensor, causal: bool,
                  softmax_scale: float):
    """Unnormalised online-softmax state (m, l, O) of rows q_rows [R, d]
    over one shard of keys k, v [N, d] (AHBM Agentic Runtime Architecture,
    §3.3 per-PE local attention; ADR-0060, §3 running state). A row that
    sees none of the shard's keys gets the identity (-inf, 0, 0)."""
    q_rows, k, v = q_rows.to(F64), k.to(F64), v.to(F64)
    R, d = q_rows.shape
    if k.shape[0] == 0:
        return (torch.full((R,), float("-inf"), dtype=F64), torch.zeros(R, dtype=F64),
                torch.zeros(R, d, dtype=F64))
    z = softmax_scale * (q_rows @ k.T)
    vis = key_visible(key_pos, row_pos, causal)
    z = z.masked_fill(~vis, float("-inf"))
    m = z.max(dim=-1).values
    empty = torch.isinf(m) & (m < 0)
    m_safe = torch.where(empty, torch.zeros_like(m), m)
    p = torch.exp(z - m_safe.unsqueeze(-1))
    return m, p.sum(-1), p @ v


def merge_states(a, b):
    """Log-sum-exp merge of two (m, l, O) states (ADR-0060 GQA fused
    attention, §4): m = max(m_a, m_b); each side is scaled by
    exp(m_side - m). exp(-inf - (-inf)) is taken as 0, so the identity
    (-inf, 0, 0) merges away (a reading: the pages leave that case open)."""
    ma, la, oa = a
    mb, lb, ob = b
    m = torch.maximum(ma, mb)
    both_empty = torch.isinf(m) & (m < 0)
    m_safe = torch.where(both_empty, torch.zeros_like(m), m)
    sa = torch.exp(ma - m_safe)
    sb = torch.exp(mb - m_safe)
    return m, la * sa + lb * sb, oa * sa.unsqueeze(-1) + ob * sb.unsqueeze(-1)


def finalize(state):
    """O = O / l once at the end, LSE = m + ln(l) (ADR-0060, §4: normalise
    once at the root; §0.5.4: N = 1 stores O / l directly)."""
    m, l, o = state
    empty = l == 0
    o_n = o / torch.where(empty, torch.ones_like(l), l).unsqueeze(-1)
    o_n = torch.where(empty.unsqueeze(-1), torch.zeros_like(o_n), o_n)
    lse = torch.where(empty, torch.full_like(m, EMPTY_LSE),
                      lse_of(m, torch.where(empty, torch.ones_like(l), l)))
    return o_n, lse
