"""Restriction of a workload's inputs to some of its branches, on the CPU.

Used by the parity tests and by the bench's CPU baseline to hand the oracle
only the branches it should compute. It moves and renumbers tensors; it
holds none of the attention arithmetic.
"""

from __future__ import annotations

import torch

from .generate import Inputs


def cpu_subset(inp: Inputs, branches) -> tuple:
    """A CPU copy of the inputs restricted to `branches` (their tokens, their
    groups' prefixes and the pages they reference, renumbered). Returns the
    subset and the list of global token ids it holds, in order."""
    qb, acc = [], 0
    for t in inp.branch_q_len:
        qb.append(acc)
        acc += t
    branches = list(branches)
    tokens = [t for b in branches for t in range(qb[b], qb[b] + inp.branch_q_len[b])]
    groups = sorted({inp.branch_group[b] for b in branches})
    gmap = {g: i for i, g in enumerate(groups)}
    ks, vs, gstart, glen, acc = [], [], [], [], 0
    for g in groups:
        s0, sl = inp.group_shared_start[g], inp.group_shared_len[g]
        ks.append(inp.k_shared[:, s0:s0 + sl].cpu())
        vs.append(inp.v_shared[:, s0:s0 + sl].cpu())
        gstart.append(acc)
        glen.append(sl)
        acc += sl
    table = inp.page_table.cpu()
    ps = inp.k_pages.shape[2]
    used = []
    for b in branches:
        npg = -(-inp.branch_private_len[b] // ps)
        used += table[b, :npg].tolist()
    uniq = sorted(set(used))
    pmap = {p: i for i, p in enumerate(uniq)}
    idx = torch.tensor(uniq, dtype=torch.int64, device=inp.k_pages.device)
    kp = inp.k_pages[idx].cpu() if uniq else inp.k_pages[:1].cpu()
    vp = inp.v_pages[idx].cpu() if uniq else inp.v_pages[:1].cpu()
    width = max(1, table.shape[1])
    new_table = torch.full((len(branches), width), -1, dtype=torch.int32)
    for i, b in enumerate(branches):
        npg = -(-inp.branch_private_len[b] // ps)
        for j in range(npg):
            new_table[i, j] = pmap[int(table[b, j])]
    tok_idx = torch.tensor(tokens, dtype=torch.int64, device=inp.q.device)
    sub = Inputs(inp.q[tok_idx].cpu(), torch.cat(ks, 1), torch.cat(vs, 1), kp, vp, new_table,
                 gstart, glen, [gmap[inp.branch_group[b]] for b in branches],
                 [inp.branch_q_len[b] for b in branches],
                 [inp.branch_private_len[b] for b in branches])
    return sub, tokens
