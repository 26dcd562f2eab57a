"""Workload descriptions: groups of branches over a shared prefix.

Vocabulary (AHBM Agentic Runtime Architecture, §1.1 and §3.1):

* a *group* owns one shared prefix of ``shared_len`` tokens, stored once;
* a *branch* (a sub-agent, or an independent request when the group's
  prefix is empty) sees ``shared prefix ++ its private suffix`` and brings
  ``q_len`` new query tokens, which are the last ``q_len`` positions of
  that context;
* private suffix tokens live in fixed-size pages reached through the
  branch's page table.

Shapes follow the Llama3-70B dimensions of ADR-0060 GQA fused attention,
§0 (H_q = 64, H_kv = 8, G = 8, d = 128).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import torch


@dataclass(frozen=True)
class Group:
    shared_len: int


@dataclass(frozen=True)
class Branch:
    group: int
    q_len: int
    private_len: int


@dataclass
class Workload:
    name: str
    dtype: str                      # "bf16" or "fp32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    groups: List[Group]
    branches: List[Branch]
    causal: bool
    seed: int
    # Per-unit split counts: one entry per group (its shared prefix) followed
    # by one entry per branch (its private suffix); 0 lets the library choose.
    splits: Optional[List[int]] = None
    # Power-of-two factor applied to Q after rounding (exact in bf16/fp32);
    # > 1 gives peaked softmax rows that make missing keys visible in O.
    q_scale: float = 1.0
    # Extra never-referenced pages in the pool (filled with random data).
    spare_pages: int = 2
    # Config-5 style: private lengths are drawn from the seed first.
    random_private: Optional[dict] = field(default=None)
    description: str = ""

    # ---- derived sizes -------------------------------------------------
    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def n_q_tokens(self) -> int:
        return sum(b.q_len for b in self.branches)

    @property
    def n_shared_tokens(self) -> int:
        return sum(g.shared_len for g in self.groups)

    def pages_of(self, b: Branch) -> int:
        return -(-b.private_len // self.page_size)

    @property
    def max_pages(self) -> int:
        return max([self.pages_of(b) for b in self.branches] + [1])

    @property
    def n_pages(self) -> int:
        return sum(self.pages_of(b) for b in self.branches) + self.spare_pages

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp32": torch.float32}[self.dtype]

    def group_shared_start(self) -> List[int]:
        out, acc = [], 0
        for g in self.groups:
            out.append(acc)
            acc += g.shared_len
        return out

    def context_len(self, b: Branch) -> int:
        return self.groups[b.group].shared_len + b.private_len

    def visible_pairs(self) -> int:
        """Number of visible (query token, key) pairs, summed over tokens."""
        total = 0
        for b in self.branches:
            c = self.context_len(b)
            for t in range(b.q_len):
                p = c - b.q_len + t
                total += (p + 1) if self.causal else c
        return total

    def flops(self) -> int:
        """Algorithmic FLOPs: 2d for Q.K plus 2d for P.V per visible
        (token, key, query head)."""
        return 4 * self.head_dim * self.num_q_heads * self.visible_pairs()

    def kv_bytes(self) -> int:
        """Unique K+V bytes: each shared prefix once, each private suffix once."""
        esz = 2 if self.dtype == "bf16" else 4
        toks = self.n_shared_tokens + sum(b.private_len for b in self.branches)
        return 2 * toks * self.num_kv_heads * self.head_dim * esz

    def io_bytes(self) -> int:
        """Q read + O written + LSE written."""
        esz = 2 if self.dtype == "bf16" else 4
        n = self.n_q_tokens * self.num_q_heads
        return 2 * n * self.head_dim * esz + 4 * n

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _llama(name, groups, branches, causal, seed, splits=None, dtype="bf16",
           page_size=16, description="", random_private=None) -> Workload:
    return Workload(name=name, dtype=dtype, num_q_heads=64, num_kv_heads=8,
                    head_dim=128, page_size=page_size, groups=groups,
                    branches=branches, causal=causal, seed=seed, splits=splits,
                    description=description, random_private=random_private)


def tiny_fp32_fanout() -> Workload:
    """Tiny fp32 fan-out: 1 KV head, G=2, d=64, 2 branches x 4 new tokens,
    shared prefix 64, private suffix 8 per branch in pages of 4, 4 shards
    per row (3 over the prefix + the suffix)."""
    return Workload(
        name="tiny_fp32_fanout", dtype="fp32", num_q_heads=2, num_kv_heads=1,
        head_dim=64, page_size=4, groups=[Group(64)],
        branches=[Branch(0, 4, 8), Branch(0, 4, 8)], causal=True, seed=1,
        splits=[3, 1, 1],
        description="tiny fp32 fan-out, 2 branches x 4 queries, prefix 64, suffix 8, pages of 4")


def decode_8k() -> Workload:
    """Llama3-70B single-layer decode: batch 1, T_q = 1, 8192 contiguous
    keys, 32 shards, attends the whole past."""
    return _llama("decode_8k", [Group(8192)], [Branch(0, 1, 0)], causal=False,
                  seed=2, splits=[32, 0],
                  description="Llama3-70B decode, 1 token over 8192 contiguous keys, 32 shards")


def fanout_8x20_32k() -> Workload:
    """Agentic fan-out: 8 sub-agents x 20 new tokens over a 32768-token
    shared prefix, 512 private tokens per branch in 16-token pages."""
    return _llama("fanout_8x20_32k", [Group(32768)],
                  [Branch(0, 20, 512) for _ in range(8)], causal=True, seed=3,
                  description="8 sub-agents x 20 tokens, shared prefix 32768, 512 private tokens each")


def prefill_32k() -> Workload:
    """Long-context causal prefill of 32768 tokens, 8 KV shards."""
    return _llama("prefill_32k", [Group(32768)], [Branch(0, 32768, 0)],
                  causal=True, seed=4, splits=[8, 0],
                  description="causal prefill of 32768 tokens, 8 shards")


def mixed_32dec_64x4() -> Workload:
    """Mixed: 32 independent decodes with KV lengths drawn from
    U{1024..65536}, plus a 64 x 4 fan-out over a 65536-token prefix with
    128 private tokens per branch."""
    g = torch.Generator().manual_seed(5)
    lens = torch.randint(1024, 65537, (32,), generator=g).tolist()
    groups = [Group(0), Group(65536)]
    branches = [Branch(0, 1, int(L)) for L in lens] + \
               [Branch(1, 4, 128) for _ in range(64)]
    return _llama("mixed_32dec_64x4", groups, branches, causal=True, seed=5,
                  random_private={"count": 32, "low": 1024, "high": 65537},
                  description="32 decodes with lengths U{1024..65536} + 64 x 4 fan-out over 65536 prefix")


def join_400_32k() -> Workload:
    """Main-agent continuation prefill after a schema-constrained join
    (AHBM Agentic Runtime Architecture, §5.4 and §5.6): 8 sub-agent results
    of 50 tokens each, 400 join-input tokens, appended in 16-token pages
    after the 32768-token shared prefix and prefilled causally (their
    queries are the whole new suffix)."""
    return _llama("join_400_32k", [Group(32768)], [Branch(0, 400, 400)], causal=True, seed=6,
                  description="join prefill: 400 join-input tokens over a 32768-token shared prefix")


def join_8000_32k() -> Workload:
    """The same after a full-text join (§5.5): 8 x 1000 = 8000 join-input
    tokens over the 32768-token shared prefix."""
    return _llama("join_8000_32k", [Group(32768)], [Branch(0, 8000, 8000)], causal=True, seed=7,
                  description="join prefill: 8000 join-input tokens over a 32768-token shared prefix")


WORKLOADS = {f.__name__: f for f in (tiny_fp32_fanout, decode_8k, fanout_8x20_32k, prefill_32k,
                                      mixed_32dec_64x4, join_400_32k, join_8000_32k)}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]()


def custom(name: str, *, dtype="bf16", H_q=16, H_kv=2, d=128, page_size=16,
           shared: Sequence[int] = (300,), branches: Sequence[tuple] = ((0, 5, 40),),
           causal=True, seed=11, splits=None, q_scale=1.0) -> Workload:
    """Small workloads for parity tests (sizes the oracle finishes quickly)."""
    return Workload(name=name, dtype=dtype, num_q_heads=H_q, num_kv_heads=H_kv,
                    head_dim=d, page_size=page_size,
                    groups=[Group(s) for s in shared],
                    branches=[Branch(*b) for b in branches], causal=causal,
                    seed=seed, splits=splits, q_scale=q_scale)
