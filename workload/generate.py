"""Seeded synthetic inputs: Q, shared K/V, paged private K/V, page tables.

Recipe (one torch.Generator seeded with the workload's seed, on the device
the tensors are made on):

1. for workloads with random private lengths, the lengths are drawn first
   (``configs.mixed_32dec_64x4`` makes the same draw);
2. Q, shared K, shared V, private K pages, private V pages are drawn from
   N(0, 1) in fp32, in that order and in fixed 16M-element chunks, then
   rounded to the storage dtype with round-to-nearest-even;
3. a random permutation of the physical page ids assigns pages to
   (branch, logical page) so that paging is not accidentally contiguous;
   the last ``spare_pages`` physical pages are never referenced.

Layouts:
  q         [n_q_tokens, H_q, d]        branch b's tokens contiguous, branches in order
  k_shared  [H_kv, n_shared_tokens, d]  groups concatenated along tokens
  v_shared  same
  k_pages   [n_pages, H_kv, page_size, d]
  v_pages   same
  page_table[n_branches, max_pages] int32, -1 padded
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import torch

from .configs import Workload

_CHUNK = 1 << 24


def _randn_(dst: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    flat = dst.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        tmp = torch.randn(e - s, generator=gen, device=dst.device, dtype=torch.float32)
        flat[s:e].copy_(tmp)          # RNE rounding to the storage dtype
    return dst


@dataclass
class Inputs:
    q: torch.Tensor
    k_shared: torch.Tensor
    v_shared: torch.Tensor
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    page_table: torch.Tensor           # int32, same device as the tensors
    group_shared_start: List[int]
    group_shared_len: List[int]
    branch_group: List[int]
    branch_q_len: List[int]
    branch_private_len: List[int]

    def to(self, device) -> "Inputs":
        f = lambda t: t.to(device)
        return Inputs(f(self.q), f(self.k_shared), f(self.v_shared), f(self.k_pages),
                      f(self.v_pages), f(self.page_table), list(self.group_shared_start),
                      list(self.group_shared_len), list(self.branch_group),
                      list(self.branch_q_len), list(self.branch_private_len))


def generate(w: Workload, device="cpu") -> Inputs:
    device = torch.device(device)
    gen = torch.Generator(device=device).manual_seed(w.seed)
    if w.random_private:
        rp = w.random_private
        torch.randint(rp["low"], rp["high"], (rp["count"],), generator=gen, device=device)
    dt = w.torch_dtype
    H_q, H_kv, d, ps = w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    q = _randn_(torch.empty(w.n_q_tokens, H_q, d, dtype=dt, device=device), gen)
    if w.q_scale != 1.0:
        q.mul_(w.q_scale)
    k_sh = _randn_(torch.empty(H_kv, w.n_shared_tokens, d, dtype=dt, device=device), gen)
    v_sh = _randn_(torch.empty(H_kv, w.n_shared_tokens, d, dtype=dt, device=device), gen)
    k_pg = _randn_(torch.empty(w.n_pages, H_kv, ps, d, dtype=dt, device=device), gen)
    v_pg = _randn_(torch.empty(w.n_pages, H_kv, ps, d, dtype=dt, device=device), gen)
    perm = torch.randperm(w.n_pages, generator=gen, device=device).cpu().tolist()
    table = torch.full((len(w.branches), w.max_pages), -1, dtype=torch.int32)
    nxt = 0
    for bi, b in enumerate(w.branches):
        for p in range(w.pages_of(b)):
            table[bi, p] = perm[nxt]
            nxt += 1
    return Inputs(q, k_sh, v_sh, k_pg, v_pg, table.to(device),
                  w.group_shared_start(), [g.shared_len for g in w.groups],
                  [b.group for b in w.branches], [b.q_len for b in w.branches],
                  [b.private_len for b in w.branches])
