"""Error contract of gqa_attn_forward, through the C ABI.

Each bad call must return the documented negative status with a message in
gqa_attn_last_error(), and launch nothing: O and LSE keep the sentinel they
were filled with. The same handle must then still give a correct forward.
Nothing here makes the GPU fault: every bad call is refused on the host
before any launch.
"""

import ctypes

import pytest
import torch

from gqa_attention_agentic_amd import _lib
from workload import custom, generate

import gpu_helpers as H
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

SENTINEL = 3.0


def _args(h, inp, causal, out_t, lse_t, splits=None, stream=None, **over):
    """gqa_attn_forward's argument list for a workload.Inputs record, with
    any pointer or size replaced by `over`."""
    ptr = lambda t: t.data_ptr() if t.numel() > 0 else None
    a = dict(q=ptr(inp.q), k_shared=ptr(inp.k_shared), v_shared=ptr(inp.v_shared),
             n_shared=inp.k_shared.shape[1], k_pages=ptr(inp.k_pages), v_pages=ptr(inp.v_pages),
             page_table=ptr(inp.page_table), max_pages=inp.page_table.shape[1],
             o=ptr(out_t), lse=ptr(lse_t))
    a.update(over)
    ng, nb = len(inp.group_shared_start), len(inp.branch_group)
    ia = _lib.int_array
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return (h._h, a["q"], a["k_shared"], a["v_shared"], a["n_shared"], a["k_pages"], a["v_pages"],
            a["page_table"], a["max_pages"], ng, ia(inp.group_shared_start), ia(inp.group_shared_len), nb,
            ia(inp.branch_group), ia(inp.branch_q_len), ia(inp.branch_private_len),
            ia(splits) if splits is not None else None, int(causal), a["o"], a["lse"], stream)


def _raw_forward(h, *args):
    st = h.lib.gqa_attn_forward(*args)
    return st, h.lib.gqa_attn_last_error().decode()


def _outputs(inp, H_q):
    out = torch.full_like(inp.q, SENTINEL)
    lse = torch.full((inp.q.shape[0], H_q), SENTINEL, dtype=torch.float32, device=inp.q.device)
    return out, lse


def _untouched(out, lse):
    torch.cuda.synchronize()
    return bool((out == SENTINEL).all()) and bool((lse == SENTINEL).all())


CASES = {
    # name: (overrides, expected status, text the message must contain)
    "q_null": (dict(q=None), _lib.GQA_ERR_INVALID_ARG, "non-NULL"),
    "o_null": (dict(o=None), _lib.GQA_ERR_INVALID_ARG, "non-NULL"),
    "lse_null": (dict(lse=None), _lib.GQA_ERR_INVALID_ARG, "non-NULL"),
    "k_shared_null": (dict(k_shared=None), _lib.GQA_ERR_INVALID_ARG, "non-NULL"),
    "page_table_null": (dict(page_table=None), _lib.GQA_ERR_INVALID_ARG, "non-NULL"),
    "k_shared_misaligned": ("k_shared+2", _lib.GQA_ERR_INVALID_ARG, "16-byte aligned"),
    "o_misaligned": ("o+8", _lib.GQA_ERR_INVALID_ARG, "16-byte aligned"),
    "lse_misaligned": ("lse+2", _lib.GQA_ERR_INVALID_ARG, "4-byte aligned"),
    "shared_extent_too_short": (dict(n_shared=999), _lib.GQA_ERR_INVALID_ARG, "n_shared_tokens"),
    "page_table_too_narrow": (dict(max_pages=2), _lib.GQA_ERR_INVALID_ARG, "max_pages_per_branch"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_rejects_bad_arguments_and_launches_nothing(case):
    w = SMALL["fanout_bf16_d128"]()      # shared prefix of 1000 tokens, suffixes of 37/50/100 (pages of 16)
    inp = generate(w, "cuda")
    h = H.handle_for(w)
    out, lse = _outputs(inp, w.num_q_heads)
    over, status, text = CASES[case]
    if isinstance(over, str):
        name, off = over.split("+")
        base = {"k_shared": inp.k_shared, "o": out, "lse": lse}[name]
        over = {name: base.data_ptr() + int(off)}
    torch.cuda.synchronize()
    st, msg = _raw_forward(h, *_args(h, inp, w.causal, out, lse, **over))
    H.say(f"  {case}: status {st}, '{msg}'")
    assert st == status, (case, st, msg)
    assert text in msg, (case, msg)
    assert _untouched(out, lse), f"{case}: the failed call wrote O or LSE"
    # the handle is still usable
    o2, l2, _ = H.run_library(w, inp, handle=h)
    ref = H.oracle_rows(w, inp)
    H.compare(w, o2, l2, ref[0], ref[1], ref[2], label=f"after {case}")
    h.close()


def test_workspace_cap_too_small_is_no_memory():
    """A plan whose partials exceed workspace_bytes_cap is refused before any
    launch (the 3-shard prefix and the suffixes need ~200 KB of partials)."""
    w = SMALL["fanout_bf16_d128"]()
    inp = generate(w, "cuda")
    h = H.handle_for(w, workspace_bytes_cap=4096)
    out, lse = _outputs(inp, w.num_q_heads)
    torch.cuda.synchronize()
    st, msg = _raw_forward(h, *_args(h, inp, w.causal, out, lse, splits=[3, 2, 2, 2]))
    H.say(f"  workspace cap: status {st}, '{msg}'")
    assert st == _lib.GQA_ERR_NO_MEMORY and "workspace_bytes_cap" in msg, (st, msg)
    assert _untouched(out, lse)
    # one shard per unit and a single unit per branch: no partials, so the cap is not reached
    solo = custom("solo", shared=(0,), branches=((0, 3, 40),), seed=130)
    si = generate(solo, "cuda")
    o2, l2, _ = H.run_library(solo, si, handle=h, splits=[0, 1])
    ref = H.oracle_rows(solo, si)
    H.compare(solo, o2, l2, ref[0], ref[1], ref[2], label="under the cap")
    h.close()


def test_capture_of_an_uncached_forward_is_refused():
    """Under HIP graph capture a forward that would plan, upload or allocate
    is refused (nothing captured); the same call outside capture works, and
    after it the capture of that call is accepted."""
    w = SMALL["fanout_bf16_d128"]()
    inp = generate(w, "cuda")
    h = H.handle_for(w)
    out, lse = _outputs(inp, w.num_q_heads)
    dummy = torch.zeros(4, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        st, msg = _raw_forward(h, *_args(h, inp, w.causal, out, lse))
        dummy.add_(1.0)
    H.say(f"  capture, uncached: status {st}, '{msg}'")
    assert st == _lib.GQA_ERR_INVALID_ARG and "capture" in msg, (st, msg)
    g.replay()
    assert _untouched(out, lse)
    del g
    o_ref, l_ref, _ = H.run_library(w, inp, handle=h)
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, capture_error_mode="thread_local"):
        st, msg = _raw_forward(h, *_args(h, inp, w.causal, out, lse))
    assert st == _lib.GQA_OK, msg
    out.fill_(SENTINEL)
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
    del g2
    h.close()
