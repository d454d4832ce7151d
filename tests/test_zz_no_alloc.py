"""moe_ffn_forward_noalloc (workspace in the library's static device array) against
moe_ffn_forward (caller workspace): the same launches with the slot-ordered combine
(MOE_FWD_DETERMINISTIC), so outputs and routing must agree bit for bit; two calls in a row, the second on a smaller batch, since the array keeps the previous
call's contents.  Sizes beyond the array are rejected on the host."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from gpu_util import DEV, Layer, say, to_dev

MID = synth.MoeShape("mid_noalloc", 16, 200, 512, 256, 32, 4, 1, 256, 4, 2)


def _both(layer, xb):
    s = layer.s
    x = to_dev(xb)
    T = x.shape[0]
    res = []
    for fn in (moe.moe_ffn_forward, moe.moe_ffn_forward_noalloc):
        ti = torch.full((T, s.top_k), -1, dtype=torch.int32, device=DEV)
        tw = torch.full((T, s.top_k), -1.0, dtype=torch.float32, device=DEV)
        sc = torch.zeros((T, s.n_experts), dtype=torch.float32, device=DEV)
        out = fn(x, layer.cfg, layer.weights, scores=sc, topk_idx=ti, topk_w=tw, deterministic=True)
        torch.cuda.synchronize()
        res.append([out.float().cpu().numpy(), ti.cpu().numpy(), tw.cpu().numpy(), sc.cpu().numpy()])
    return res


@pytest.mark.parametrize("shape", [synth.TINY, MID])
def test_noalloc_matches_forward_twice(shape):
    say(f"noalloc forward {shape.name}: T={shape.tokens}, then T=37")
    layer = Layer(shape)
    xb = synth.gen_x(shape)
    for rows in (xb, xb[11:48]):
        ref, got = _both(layer, np.ascontiguousarray(rows))
        for a, b in zip(ref, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_rejects_sizes_beyond_the_array():
    say("noalloc forward: T beyond the static array")
    layer = Layer(synth.TINY)
    cfg = moe.MoeConfig.of(synth.V3_DECODE)
    assert moe.moe_ffn_workspace_size(223, cfg) <= moe._lib.MOE_NOALLOC_SCRATCH_BYTES < moe.moe_ffn_workspace_size(224, cfg)
    big = torch.zeros((100000, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_ffn_forward_noalloc(big, layer.cfg, layer.weights)
    assert e.value.status == moe._lib.MOE_ERR_WORKSPACE
