"""moe_forward_static (the entry point that allocates nothing: its workspace
is the library's static per-GPU array) against moe_forward with a
torch-allocated workspace, through the C ABI: identical output bits on two
calls in a row, the second with a smaller batch (so stale intermediates of
the first call sit in the array), plus the synchronous rejection of a
problem too large for the array."""
import ctypes

import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth

pytestmark = pytest.mark.gpu


def _run_pair(cfg):
    inp = moe_synth.make_inputs(cfg, "cuda")
    p = moe.Problem.from_config(cfg)
    assert moe.workspace_size(p) <= moe.STATIC_SCRATCH_BYTES
    layer = moe.MoeLayer(p, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"])
    want = layer(inp["hidden"], inp["topk_ids"], inp["topk_weights"], None, inp["is_padding"],
                 inp["expert_num_tokens"], inp["eplb"])
    got = torch.full((cfg.T, cfg.K), 0x7FBF, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    moe.forward_static(p, inp["hidden"], inp["topk_ids"], inp["topk_weights"], inp["w13"],
                       inp["w13_sf"], inp["w2"], inp["w2_sf"], got, inp["is_padding"],
                       inp["expert_num_tokens"], inp["eplb"])
    torch.cuda.synchronize()
    return torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_static_forward_matches_forward():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    first = moe_synth.custom(name="static_a", T=200, E=16, top_k=4, K=1024, N=768, seed=71,
                             routing="zipf", zipf_s=1.1, pad_frac=0.05)
    second = moe_synth.custom(name="static_b", T=48, E=16, top_k=4, K=1024, N=768, seed=72)
    assert _run_pair(first), "first call differs from moe_forward"
    assert _run_pair(second), "second (smaller) call differs from moe_forward"
    # decode-shaped, block fp8 and MX: the same bits as moe_forward
    decode = moe_synth.custom(name="static_decode", T=64, E=64, top_k=8, K=2048, N=1024,
                              seed=73, act_quant="mxfp8", weight_quant="mxfp4")
    assert _run_pair(decode), "MX decode-shaped call differs from moe_forward"


def test_static_forward_rejects_oversized():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib = moe.load_library()
    p = moe.Problem(8192, 7168, 2048, 256, 8)
    assert moe.workspace_size(p) > moe.STATIC_SCRATCH_BYTES
    out = torch.empty(16, dtype=torch.uint8, device="cuda")
    ptr = ctypes.c_void_p(out.data_ptr())
    st = lib.moe_forward_static(ctypes.byref(p.c()), ptr, None, ptr, ptr, None, None, ptr, ptr,
                                ptr, ptr, ptr, None)
    assert st == -3 and "static scratch" in lib.moe_last_error().decode()
