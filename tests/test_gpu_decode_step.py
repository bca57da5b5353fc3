"""GPU parity of the decode-step stack (the timing harness's workload).

Two layers of the 36-layer batch-1 stack, four dependent svq_linear_batched
calls per layer, every layer with its own matrices.  The outputs of an eager
pass are checked against the CPU oracle within the output tolerance (and the
tighter bound of the exact decode path); the same calls captured into one HIP
graph are then replayed several times, with eager work and synchronisations
between the replays, and every replay must reproduce the eager outputs bit
for bit (the batch-1 path reduces every output row inside one workgroup in a
fixed order).
"""
import numpy as np
import pytest

import synth
from oracle import svq_oracle as so
from tests.gpu_common import assert_within_tolerance, out_to_f64, require_gpu, torch

pytestmark = pytest.mark.gpu


def _build(svq, stack, stream):
    calls, outs, refs = [], [], []
    for mats, xs in stack:
        pms = [svq.pack(w) for w in mats]
        for c, idx in enumerate(synth.DECODE_CALLS):
            x = torch.from_numpy(xs[c].view(np.int16)).view(torch.bfloat16).cuda()
            ys = [torch.empty((1, mats[j].n), dtype=torch.float32, device="cuda") for j in idx]
            calls.append(svq.BatchedCall([pms[j] for j in idx], [x] * len(idx), ys, stream=stream))
            outs += ys
            refs += [(mats[j], xs[c]) for j in idx]
    return calls, outs, refs


def test_decode_step_eager_and_graph_replays():
    svq = require_gpu()
    stack = synth.decode_stack(2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    calls, outs, refs = _build(svq, stack, side)
    assert len(calls) == 8 and len(outs) == 14

    def step():
        for call in calls:
            call()

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (mat, x), o in zip(refs, eager):
        y64, W = so.linear_from_inputs(mat, x)
        y = out_to_f64(o)
        assert_within_tolerance(y, y64, x, W, label=f"decode step {mat.name}")
        assert_within_tolerance(y, y64, x, W, rel=1e-3, label=f"decode step exact {mat.name}")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        for (mat, _), o, e in zip(refs, outs, eager):
            assert torch.equal(o, e), f"replay {rep}: {mat.name} differs from the eager pass"


def test_first_token_pass_two_layers():
    """The first-token leg: two layers of the stack over a 128-token prompt
    (every call at m = 128, the prefill path), checked against the oracle
    within the output tolerance; graph replays reproduce the eager pass."""
    svq = require_gpu()
    stack = synth.decode_stack(2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    P = synth.PREFILL_TOKENS
    calls, outs, refs = [], [], []
    for layer, (mats, _) in enumerate(stack):
        pms = [svq.pack(w) for w in mats]
        xs = synth.prompt_activations(layer, synth.call_input_widths(mats), P)
        for c, idx in enumerate(synth.DECODE_CALLS):
            x = torch.from_numpy(xs[c].view(np.int16)).view(torch.bfloat16).cuda()
            ys = [torch.empty((P, mats[j].n), dtype=torch.float32, device="cuda") for j in idx]
            calls.append(svq.BatchedCall([pms[j] for j in idx], [x] * len(idx), ys, stream=side))
            outs += ys
            refs += [(mats[j], xs[c]) for j in idx]

    def step():
        for call in calls:
            call()

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (mat, x), o in zip(refs, eager):
        y64, W = so.linear_from_inputs(mat, x)
        assert_within_tolerance(out_to_f64(o), y64, x, W, label=f"first token {mat.name}")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        for (mat, _), o, e in zip(refs, outs, eager):
            assert torch.equal(o, e), f"replay {rep}: {mat.name} differs from the eager pass"
