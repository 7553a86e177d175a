"""The small configurations captured into HIP graphs and replayed.

The 768 -> 768 Linear forward step (delayed scaling) and the BERT-base-shaped layer
step (current scaling, shared quantization) are captured once and replayed several
times, with unrelated eager work and synchronizations between replays; every replay
must reproduce the eager run of the same step bit for bit (codes, outputs, amax
history, scales).  This checks that the library's launches are capture-safe: no
allocation, no host synchronization and no memset node inside a step.
"""

import pytest
import torch

from fp8_precision_transformer_amd.shapes import BERT_BASE
from fp8_precision_transformer_amd.steps import LayerStep, LinearForwardStep, capture

from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _snapshot(step):
    return {k: v.clone() for k, v in step.outputs().items()}


def _check(step, ref, tag):
    for k, v in step.outputs().items():
        assert torch.equal(v, ref[k]), f"{tag}: {k} differs from the eager step"


def test_linear_step_graph_replays_match_eager():
    st = torch.cuda.Stream()
    step = LinearForwardStep(st)
    step.run()                      # first call on the stream: workspace and caches
    torch.cuda.synchronize()
    step.reset()
    refs = []
    for _ in range(4):              # the delayed-scaling state advances every step
        step.run()
        st.synchronize()
        refs.append(_snapshot(step))
    step.reset()
    torch.cuda.synchronize()
    g = capture(step)
    step.reset()
    torch.cuda.synchronize()
    for i in range(4):
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        noise = torch.randn(4096, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        _check(step, refs[i], f"replay {i}")


def test_bert_layer_step_graph_replays_match_eager():
    st = torch.cuda.Stream()
    step = LayerStep(BERT_BASE, st)
    step.run()
    st.synchronize()
    ref = _snapshot(step)
    for k in list(step.outputs()):  # clear the outputs so a replay that writes nothing fails
        v = step.outputs()[k]
        v.zero_() if v.dtype != torch.float32 else v.fill_(float("nan"))
    torch.cuda.synchronize()
    g = capture(step)
    for i in range(3):
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        torch.cuda.synchronize()
        _check(step, ref, f"replay {i}")
        for k in list(step.outputs()):
            v = step.outputs()[k]
            v.zero_() if v.dtype != torch.float32 else v.fill_(float("nan"))
        torch.cuda.synchronize()
