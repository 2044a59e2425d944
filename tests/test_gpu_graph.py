"""HIP graph capture of the layer (needs an MI355X): the C entry points make
no allocation, memset or synchronisation, so a whole step records into a
graph. Every replay, with eager work and synchronisations between replays,
must give the eager result bit for bit (the kernels are deterministic)."""
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["worked_example_geometry", "skewed_small"])
def test_forward_graph_replays_match_eager(name):
    w = (wl.WORKLOADS[name] if name in wl.WORKLOADS else
         wl.Workload("skewed_small", T=700, D=256, E=32, k=4, I=192, zipf_s=1.5,
                     return_logits=True, I_shared=128))
    inp = wl.make_inputs(w, seed=4)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                      I_shared=w.I_shared)
    lay = moe.LayerForward(d, g["w_router"], g["w_gate_up"], g["w_down"],
                           logit_bias=g["logit_bias"], shared_gate_up=g["shared_gate_up"],
                           shared_down=g["shared_down"], want_logits=w.return_logits)
    outs = lambda: [t.clone() for t in (lay.out, lay.topk_idx, lay.topk_w, lay.counts,  # noqa
                                        lay.offsets, lay.pos) + ((lay.logits,) if lay.logits
                                                                  is not None else ())]
    lay(g["x"])
    torch.cuda.synchronize()
    ref = outs()
    graph = _capture(lambda: lay(g["x"]))
    other = torch.randn_like(g["x"].float()).to(g["x"].dtype)
    for i in range(4):
        lay.out.fill_(0)
        lay.topk_idx.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {i}"
        lay(other)  # eager work between replays, on other inputs
        torch.cuda.synchronize()


def test_training_step_graph_replays_match_eager():
    w = wl.Workload("train_graph", T=512, D=256, E=8, k=2, I=192, I_shared=64)
    inp = wl.make_inputs(w, seed=5)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, I_shared=w.I_shared)
    lay = moe.LayerTrain(d, g["w_router"], g["w_gate_up"], g["w_down"],
                         shared_gate_up=g["shared_gate_up"], shared_down=g["shared_down"])
    dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(6)).to(
        torch.bfloat16).cuda()

    def step():
        lay.forward(g["x"])
        lay.backward(dout)

    grads = lambda: [t.clone() for t in (lay.out, lay.dx, lay.dw_router, lay.dw_gate_up,  # noqa
                                         lay.dw_down, lay.dw_shared_gate_up,
                                         lay.dw_shared_down)]
    step()
    torch.cuda.synchronize()
    ref = grads()
    graph = _capture(step)
    for i in range(3):
        lay.dw_gate_up.fill_(0)
        lay.dx.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, grads()):
            assert torch.equal(a, b), f"replay {i}"
        lay.forward(torch.randn_like(g["x"].float()).to(torch.bfloat16))
        torch.cuda.synchronize()
