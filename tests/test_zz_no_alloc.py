"""The no-allocation forward (moe_ffn_forward_noalloc: the inference forward
whose scratch is the library's own per-GPU device array, for callers that
cannot allocate) against moe_ffn_forward with a caller workspace: bit for bit
on two calls in a row, the second with a smaller input, so the second call
runs on an array that still holds the first call's contents."""
import pytest
import torch

from sparse_mixture_experts_route_amd import _lib as L
from workloads import WORKLOADS, make_inputs

from gpu_helpers import make_layer, need_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc(layer, x):
    s = layer.last
    out = torch.full_like(x, float("nan"))
    L.moe_ffn_forward_noalloc(layer._shape_T(x.shape[0]), layer.weights, x, None, s["offsets"], s["perm"], s["pos"],
                              s["weights"], s["gate"], out)
    return out


def test_noalloc_forward_equals_forward_twice_second_smaller():
    need_gpu()
    base = WORKLOADS["qwen2moe"]
    # 512 tokens: routed weight streams with the split bf16 activation, the
    # shared expert on the 256x256 kernel with its down projection split eight
    # ways along K (about 58.5 MiB of the 64 MiB array on a 256-CU device);
    # 48 tokens: every GEMM a weight stream
    for T in (512, 48):
        w = base.with_(T=T, seed=60 + T)
        inp = make_inputs(w, device="cuda")
        layer = make_layer(w, inp, fuse_gather=True)
        ref = layer.forward(inp["x"], save=False)
        out = _noalloc(layer, inp["x"])
        torch.cuda.synchronize()
        say(f"T={T}: no-allocation forward equals the forward bit for bit: {torch.equal(out, ref)}")
        assert torch.equal(out, ref), f"T={T}"


def test_noalloc_rejects_sizes_beyond_its_array():
    need_gpu()
    w = WORKLOADS["qwen2moe"].with_(T=2048)
    sh = L.make_shape(w.T, w.H, w.E, w.k, w.I, w.Is, w.score, w.renorm, w.shared_gated, L.DTYPE_BF16)
    assert L.workspace_bytes(sh, L.OP_FFN_FORWARD) > 64 << 20
    x = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MoeError) as e:
        L.moe_ffn_forward_noalloc(sh, L.weights_struct(x, x), x, None, x, x, x, x, None, x)
    assert e.value.status == L.MOE_EWORKSPACE
