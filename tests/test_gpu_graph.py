"""Forward calls captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

Every path enqueues only kernels, on the caller's stream, into caller-owned
buffers (no allocation, copy or memset inside a call), so a captured call replays
exactly the launches it recorded. Each case replays the graph several times with
eager work between the replays (outputs overwritten with NaN, and from the third
replay on new inputs written into the same buffers) and checks every replay
bitwise against an eager call on the same inputs; kda_fwd_noalloc, the entry point
for callers that cannot allocate, is captured too.
"""
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads

pytestmark = pytest.mark.gpu

# kda_fwd_noalloc runs only the single pass and the token-by-token path
CASES = [
    ("fused", [512] * 6, 4, False),
    ("fused", [512] * 6, 4, True),
    ("segmented", [2048], 4, False),
    ("split", [300, 200], 2, False),
    ("recurrent", [1] * 64, 4, False),
    ("recurrent", [1] * 64, 4, True),
]


@pytest.mark.parametrize("path,lens,H,noalloc", CASES)
def test_captured_call_replays_match_eager(gpu, path, lens, H, noalloc):
    print(f"\n[case] graph capture: {path}, {len(lens)} sequences, H={H}, noalloc={noalloc}", flush=True)
    w = workloads.make(lens, H, seed=200 + len(lens), init_std=0.02)
    stream = torch.cuda.Stream(gpu)
    q, k, v, g, b = (t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    cu = w.cu_seqlens().to(gpu)
    s0 = w.initial_state.to(gpu)
    torch.cuda.synchronize(gpu)
    call = kda.prepare_call(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path=path,
                            stream=stream, no_workspace=noalloc)
    run = call.run_noalloc if noalloc else call.run

    def eager():
        with torch.cuda.stream(stream):
            run()
        stream.synchronize()
        return call.out.clone(), call.final_state.clone()

    def scribble():
        with torch.cuda.stream(stream):
            call.out.fill_(float("nan"))
            call.final_state.fill_(float("nan"))
        stream.synchronize()

    ref = eager()  # also the first call, before any capture
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run()
    gen = torch.Generator(device="cpu").manual_seed(300 + len(lens))
    for rep in range(5):
        if rep >= 2:  # new inputs in the same buffers, and their eager result
            for t in (q, k, v):
                t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype).to(gpu))
            torch.cuda.synchronize(gpu)
            ref = eager()
        scribble()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        assert torch.equal(call.out, ref[0]), f"replay {rep}: outputs differ from the eager call"
        assert torch.equal(call.final_state, ref[1]), f"replay {rep}: final states differ from the eager call"
        assert torch.isfinite(call.out.float()).all()
