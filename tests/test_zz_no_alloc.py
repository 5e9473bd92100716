"""flint_moe_forward_static, the entry point that allocates nothing (its
workspace is the library's own static device scratch), against
flint_moe_forward with a caller-allocated workspace: the same bits, on two
calls in a row where the second has fewer tokens (the scratch keeps the first
call's contents), on the decode and on the tiled kernels; the second call's
outputs also against the oracle; and the call captured in a HIP graph (which
refuses allocations during capture) replayed against eager calls."""
import numpy as np
import pytest
import torch

import gpu_common as G
from oracle import oracle as orc
from routed_expert_ffn_flint_amd import api, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    yield
    torch.cuda.synchronize()


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _static_and_workspace(d, w, x):
    ref = api.forward(d, x, w, return_routing=True)  # a torch-allocated workspace
    got = [torch.full_like(r, -1) for r in ref]
    api.flint_moe_forward_static(d, x, w, *got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("name,T1,T2", [("decode32", 32, 8), ("prefill4096", 600, 200)])
def test_static_entry_point_matches_workspace_entry_point(name, T1, T2):
    wl = inputs.WORKLOADS[name]
    d = api.dims_of(wl)
    w = inputs.make_layer(wl, 0, "cuda")
    x = inputs.make_tokens(wl, T=T1, device="cuda")
    print(f"no-alloc: {name} T={T1} then T={T2}", flush=True)
    for T in (T1, T2):
        xt = x[:T].contiguous()
        ref, got = _static_and_workspace(d, w, xt)
        for r, g in zip(ref, got):
            assert _same(r, g), f"{name} T={T}: static-scratch call differs from the workspace call"
    # the second (smaller) call against the oracle, on every token
    out, idx, tw = got
    od = G.oracle_dims(wl)
    xh = inputs.to_numpy_f32(xt)
    router, bias = inputs.to_numpy_f32(w["router"]), inputs.to_numpy_f32(w.get("bias"))
    o_idx, o_w, tie = orc.route(od, xh, router, bias)
    gi = idx.cpu().numpy()
    G.check_routing(gi, tw.cpu().numpy(), o_idx, o_w, tie, f"{name} static", G.scores_fn(od, xh, router, bias))
    ref_out, _, _, _ = orc.forward(od, xh, G.host_weights(w, set(gi.ravel().tolist())), force_idx=gi)
    G.check_output(out.cpu().numpy(), ref_out, f"{name} static")


def test_static_entry_point_captured_in_a_graph():
    wl = inputs.WORKLOADS["decode32"]
    d = api.dims_of(wl)
    w = inputs.make_layer(wl, 0, "cuda")
    wst = api.weights_struct(d, w)
    x = inputs.make_tokens(wl, device="cuda")
    x2 = inputs.make_tokens(wl, T=16, device="cuda", stream=1)
    refs = list(api.forward(d, x, w, return_routing=True))
    outs = [torch.empty_like(r) for r in refs]
    api.flint_moe_forward_static(d, x, wst, *outs)  # first call on the device: scratch looked up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.flint_moe_forward_static(d, x, wst, *outs, stream=s)
    torch.cuda.synchronize()
    other = [torch.empty((16, wl.hidden), dtype=torch.float32, device="cuda"),
             torch.empty((16, wl.top_k), dtype=torch.int32, device="cuda"),
             torch.empty((16, wl.top_k), dtype=torch.float32, device="cuda")]
    for r in range(3):
        api.flint_moe_forward_static(d, x2, wst, *other)  # an eager call dirties the scratch
        for o in outs:
            o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert _same(o, ref), f"replay {r} differs"
