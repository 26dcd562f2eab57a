"""Helpers for the GPU parity tests: run the HIP library, run the oracle on
CPU copies of the same inputs, compare to the tolerance of the workload's
dtype."""

from __future__ import annotations

import sys

import torch

import oracle
from workload import cpu_subset, generate  # noqa: F401  (cpu_subset: re-exported for the tests)
from workload.generate import Inputs  # noqa: F401

# Tolerances on O (over all compared elements): bf16 max-abs 2e-2 and
# mean-abs 2e-3; fp32 max-abs 1e-4. LSE is checked too (1e-3 bf16, 1e-4 fp32):
# at long contexts O alone moves little when a whole unit of keys is lost.
TOL = {"bf16": dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3),
       "fp32": dict(o_max=1e-4, o_mean=1e-4, lse_max=1e-4)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def handle_for(w, **kw):
    from gqa_attention_agentic_amd import GqaAttention
    return GqaAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.dtype, **kw)


def run_library(w, inp, splits="workload", handle=None, causal=None):
    h = handle or handle_for(w)
    sp = w.splits if splits == "workload" else splits
    o, lse = h.forward_inputs(inp, w.causal if causal is None else causal, splits=sp)
    torch.cuda.synchronize()
    return o, lse, h


def oracle_rows(w, inp, branches=None, tokens=None, heads=None):
    """Oracle O / LSE for `tokens` (global ids; default all) of `branches`."""
    if branches is None:
        branches = range(len(inp.branch_q_len))
    sub, tok_ids = cpu_subset(inp, branches)
    if tokens is None:
        tokens = tok_ids
    pos = {t: i for i, t in enumerate(tok_ids)}
    o, lse = oracle.attention(sub, w.num_kv_heads, w.page_size, w.causal,
                              tokens=[pos[t] for t in tokens], heads=heads)
    return o, lse, list(tokens)


def compare(w, o_gpu, lse_gpu, o_ref, lse_ref, tokens, heads=None, label=""):
    tol = TOL[w.dtype]
    tk = torch.tensor(tokens, dtype=torch.int64, device=o_gpu.device)
    og = o_gpu[tk].double().cpu()
    lg = lse_gpu[tk].double().cpu()
    if heads is not None:
        hh = torch.tensor(heads, dtype=torch.int64)
        og, lg = og[:, hh], lg[:, hh]
    assert torch.isfinite(og).all(), f"{label}: non-finite O"
    err = (og - o_ref).abs()
    lerr = (lg - lse_ref).abs()
    stats = dict(o_max=err.max().item(), o_mean=err.mean().item(), lse_max=lerr.max().item())
    say(f"  {label}: {stats}")
    assert stats["o_max"] <= tol["o_max"], (label, stats)
    assert stats["o_mean"] <= tol["o_mean"], (label, stats)
    assert stats["lse_max"] <= tol["lse_max"], (label, stats)
    return stats


def full_parity(w, splits="workload", label=None, inp=None):
    label = label or w.name
    say(f"[parity] {label}: generating")
    inp = inp or generate(w, "cuda")
    say(f"[parity] {label}: library")
    o, lse, h = run_library(w, inp, splits=splits)
    say(f"[parity] {label}: oracle")
    o_ref, l_ref, toks = oracle_rows(w, inp)
    return compare(w, o, lse, o_ref, l_ref, toks, label=label), h
