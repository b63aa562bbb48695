"""The allocation-free layer entry point (qmoe_layer_noalloc, workspace in the
library's fixed device scratch) against qmoe_layer with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller input, on both
paths; a call beyond the scratch is refused before anything runs; and the
call captured in a HIP graph replays to the eager result."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import Layer, rel_l2, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
E, H, F, K = 32, 1024, 512, 8


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm.load()
    lay = Layer(E, H, F, seed=4242)
    yield lay
    torch.cuda.synchronize()


def _inputs(T, seed, dtype):
    g = synth.generator(seed)
    x = synth.rand_x(g, (T, H))
    ids, w = synth.route_topk_fast(synth.normal_logits(g, T, E), K)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x.to(DEV), ids.to(DEV), w.to(DEV)


def _compare(got, want, dtype):
    if dtype == "bf16":
        # same kernels, fixed summation order: identical
        assert torch.equal(got, want)
    else:
        # the f32 down projection adds its k expert terms with atomics, so the
        # summation order (and the last bits) may differ from call to call
        err = rel_l2(got.cpu().numpy(), want.cpu().numpy())
        assert err <= 1e-6, err
        assert np.allclose(got.cpu().numpy(), want.cpu().numpy(), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_layer_two_calls(layer, dtype):
    for T, seed in ((48, 1), (5, 2)):            # second call smaller
        say(f"noalloc {dtype} T={T}")
        x, ids, w = _inputs(T, seed, dtype)
        want = qm.qmoe_layer(layer.dev, x, ids, w)
        out = torch.full((T, H), float("nan"), device=DEV)
        got = qm.qmoe_layer_noalloc(layer.dev, x, ids, w, out=out)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        _compare(got, want, dtype)


def test_noalloc_refuses_beyond_scratch(layer):
    say("noalloc beyond scratch")
    T = 20000
    need = layer.dev.workspace_bytes(T, K, qm.QMOE_BF16)
    assert need > qm.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(T, K, dtype=torch.int32, device=DEV)
    w = torch.zeros(T, K, dtype=torch.float32, device=DEV)
    out = torch.full((T, H), 7.0, device=DEV)
    with pytest.raises(qm.QmoeError) as ei:
        qm.qmoe_layer_noalloc(layer.dev, x, ids, w, out=out)
    assert ei.value.status == 9
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())          # nothing ran


def test_noalloc_graph_replays(layer):
    say("noalloc graph capture")
    T = 16
    x, ids, w = _inputs(T, 3, "f32")
    want = qm.qmoe_layer(layer.dev, x, ids, w)
    out = torch.empty(T, H, device=DEV)
    qm.qmoe_layer_noalloc(layer.dev, x, ids, w, out=out)     # first call: set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        qm.qmoe_layer_noalloc(layer.dev, x, ids, w, out=out)
    for rep in range(3):
        out.fill_(float("nan"))
        # eager work between replays, on the same scratch
        x2, i2, w2 = _inputs(7, 10 + rep, "f32")
        qm.qmoe_layer_noalloc(layer.dev, x2, i2, w2)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), rep
        _compare(out, want, "f32")
