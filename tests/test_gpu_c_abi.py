"""The C ABI from plain C: tests/c_abi/forward_from_c.c (built by build())
reads a problem's inputs from files, runs moe_forward with hipMalloc'd
buffers on the default stream, and writes the output.  Its output must meet
the oracle's bound and equal the Python binding's moe_forward bit for bit
(the same library, called without torch in the process)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import moe_synth
import test_gpu_parity as P
from parity_util import check_output, to_np
from test_gpu_parity import gpu  # noqa: F401  (the session fixture)

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "forward_from_c")

CASES = {
    "c_tiny": moe_synth.CONFIGS["tiny"],
    # several tiles, a ragged tail, padding tokens and skewed routing: the
    # second (256-row) tile list runs on the library's own stream
    "c_skewed": moe_synth.custom(name="c_skewed", T=256, E=8, top_k=3, K=1024, N=1024,
                                 seed=91, routing="zipf", zipf_s=1.1, pad_frac=0.05),
}


def _write(path, t):
    a = t.cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    a.tofile(path)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_from_plain_c(gpu, name, tmp_path, monkeypatch):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with __graft_entry__.build()")
    for k in ("MOE_TILE_M", "MOE_KSPLIT", "MOE_TALL", "MOE_KROT"):
        monkeypatch.delenv(k, raising=False)
    cfg = CASES[name]
    P.CASES[cfg.name] = cfg
    _, h, dev, ref = P.case(cfg.name)
    d = str(tmp_path)
    _write(os.path.join(d, "hidden.bin"), dev["hidden"].view(torch.int16))
    _write(os.path.join(d, "topk_ids.bin"), dev["topk_ids"].to(torch.int32))
    _write(os.path.join(d, "topk_w.bin"), dev["topk_weights"].to(torch.float32))
    if dev["is_padding"] is not None:
        _write(os.path.join(d, "is_padding.bin"), dev["is_padding"].to(torch.uint8))
    _write(os.path.join(d, "w13.bin"), dev["w13"].view(torch.uint8))
    _write(os.path.join(d, "w13_sf.bin"), dev["w13_sf"].to(torch.float32))
    _write(os.path.join(d, "w2.bin"), dev["w2"].view(torch.uint8))
    _write(os.path.join(d, "w2_sf.bin"), dev["w2_sf"].to(torch.float32))
    args = [EXE, d, str(cfg.T), str(cfg.E), str(cfg.top_k), str(cfg.K), str(cfg.N)]
    print(" ".join(args), flush=True)
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    print(res.stdout + res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    got = np.fromfile(os.path.join(d, "out.bin"), dtype=np.uint16).reshape(cfg.T, cfg.K)
    check_output(got, ref["out"], f"{name} from C")
    want = to_np(P.run_forward(cfg, dev))
    assert np.array_equal(got, want), f"{name}: the C caller's output differs from the binding's"
