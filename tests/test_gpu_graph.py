"""A forward whose plan is cached issues only kernel launches (and, for a
plan that runs the two attention kernels side by side, the fork / join
events of the handle's side stream): no allocation, no upload, no memset.
Such a forward is captured into a HIP graph and replayed several times,
with the program's own eager work and synchronisations between the
replays; every replay must equal the eager result bit for bit."""

import pytest
import torch

from workload import generate

import gpu_helpers as H
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["fanout_bf16_d128", "decode_bf16", "mixed_bf16", "tiny_fp32_fanout"])
def test_cached_forward_replays_in_a_graph(name):
    w = SMALL[name]()
    H.say(f"[graph] {name}")
    inp = generate(w, "cuda")
    h = H.handle_for(w)
    out = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[0], w.num_q_heads, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # eager: plan upload, workspace, counter clear, then a cached forward
        for _ in range(2):
            h.forward_inputs(inp, w.causal, splits=w.splits, out=out, lse=lse, stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        h.forward_inputs(inp, w.causal, splits=w.splits, out=out, lse=lse,
                         stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"replay {rep}: O differs"
        assert torch.equal(lse, l_ref), f"replay {rep}: LSE differs"
        # eager work between replays on the same handle and buffers
        h.forward_inputs(inp, w.causal, splits=w.splits, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref)
    del g
    h.close()


def test_graph_stays_valid_after_forwards_with_other_metadata():
    """A graph captured from a cached forward keeps its plan, counters and
    workspace: later eager forwards on the same handle with other metadata --
    a smaller plan, then one whose partials need a larger workspace -- get
    buffers of their own, and the graph still replays bit-identically."""
    wa = SMALL["fanout_bf16_d128"]()             # H_q 16, H_kv 2, d 128, pages of 16
    wb = SMALL["decode_bf16"]()                  # same head geometry, 8-shard decode
    wc = SMALL["prefill_bf16"]()                 # 700-token prefill in 3 shards: more partials
    ia, ib, ic = generate(wa, "cuda"), generate(wb, "cuda"), generate(wc, "cuda")
    h = H.handle_for(wa)
    out = torch.empty_like(ia.q)
    lse = torch.empty(ia.q.shape[0], wa.num_q_heads, dtype=torch.float32, device="cuda")
    h.forward_inputs(ia, wa.causal, splits=wa.splits, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        h.forward_inputs(ia, wa.causal, splits=wa.splits, out=out, lse=lse,
                         stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    refs = {}
    for rep in range(3):
        for w, inp in ((wb, ib), (wc, ic)):
            o, l, _ = H.run_library(w, inp, handle=h)
            if w.name in refs:
                assert torch.equal(o, refs[w.name][0]) and torch.equal(l, refs[w.name][1]), w.name
            else:
                ref = H.oracle_rows(w, inp)
                H.compare(w, o, l, ref[0], ref[1], ref[2], label=f"{w.name} between replays")
                refs[w.name] = (o.clone(), l.clone())
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"replay {rep}: O differs"
        assert torch.equal(lse, l_ref), f"replay {rep}: LSE differs"
    del g
    h.close()
