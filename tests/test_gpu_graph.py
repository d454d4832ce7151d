"""The forward under HIP graph capture.  moe_ffn_forward (caller workspace) and
moe_ffn_forward_noalloc (the library's static array) enqueue only kernels on the caller's stream:
no allocation, no host synchronisation, no memset node.  torch can therefore capture one call into
a graph.  Each replay, with a new input copied into the captured buffer beforehand and an eager
forward plus stream synchronisations between replays, must equal the eager forward on the same
input bit for bit (output and routing).  Shapes: the weight-streaming GEMM (tiny), 64-row tiles
(mid_a) and 128-row tiles (mid_b)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from gpu_util import DEV, Layer, say, to_dev

MID_A = synth.MoeShape("mid_a", 10, 200, 512, 256, 32, 4, 1, 256, 4, 2)
MID_B = synth.MoeShape("mid_b", 11, 1024, 384, 256, 16, 4, 1, 384, 4, 4)


def _eager(layer, x):
    s = layer.s
    T = x.shape[0]
    ti = torch.empty((T, s.top_k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, s.top_k), dtype=torch.float32, device=DEV)
    out = moe.moe_ffn_forward(x, layer.cfg, layer.weights, topk_idx=ti, topk_w=tw)
    torch.cuda.synchronize()
    return out, ti, tw


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("shape", [synth.TINY, MID_A, MID_B], ids=lambda s: s.name)
def test_forward_graph_replays_match_eager(shape, noalloc):
    say(f"forward captured in a HIP graph: {shape.name}, {'noalloc' if noalloc else 'caller workspace'}")
    layer = Layer(shape)
    s = shape
    T = s.tokens
    inputs = [to_dev(synth.gen_x(s, tensor_id=t)) for t in (synth.T_X, 90, 91)]
    x_buf = inputs[0].clone()
    out_buf = torch.empty_like(x_buf)
    ti_buf = torch.empty((T, s.top_k), dtype=torch.int32, device=DEV)
    tw_buf = torch.empty((T, s.top_k), dtype=torch.float32, device=DEV)
    ws = None if noalloc else moe.alloc_workspace(T, layer.cfg, DEV)

    def call():
        if noalloc:
            moe.moe_ffn_forward_noalloc(x_buf, layer.cfg, layer.weights, out=out_buf, topk_idx=ti_buf, topk_w=tw_buf)
        else:
            moe.moe_ffn_forward(x_buf, layer.cfg, layer.weights, workspace=ws, out=out_buf, topk_idx=ti_buf,
                                topk_w=tw_buf)

    # a warm-up call on a side stream (torch's recommended practice before capture; it also looks
    # up the static array's device address outside the capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep, x in enumerate(inputs + inputs[::-1]):
        x_buf.copy_(x)
        out_buf.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out_buf.clone(), ti_buf.clone(), tw_buf.clone())
        ref = _eager(layer, x)
        for name, a, b in zip(("out", "topk_idx", "topk_w"), got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rep, name)
        say(f"  replay {rep}: equal to the eager forward")
    del graph
    torch.cuda.synchronize()
