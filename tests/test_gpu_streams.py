"""The two-list GEMM steps' second stream, seen from the caller.

moe_forward (and the GEMM entry points) run the 256-row tile list's launches
on a stream the library keeps per device, forked from the caller's stream
and joined back to it with events.  Two things follow that the parity tests
do not show: a HIP graph captured from the caller's stream contains the
forked launches (every replay gives the eager bits), and host threads that
call the library at the same time on their own streams still get their own
results (the fork-launch-join sequence is kept whole by a per-device lock).
"""
import threading

import pytest
import torch

import fp8_block_quantized_group_amd as moe
from test_gpu_parity import case, gpu, problem  # noqa: F401  (gpu: the session fixture)

pytestmark = pytest.mark.gpu

NAME = "tall_ue8m0"


def _args(dev):
    return dict(is_padding=dev["is_padding"], expert_num_tokens=dev["expert_num_tokens"])


def _forward(p, cfg, dev, out, ws):
    moe.forward(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], dev["w13"],
                dev["w13_sf"], dev["w2"], dev["w2_sf"], out, ws, **_args(dev))


def _setup(monkeypatch):
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    monkeypatch.delenv("MOE_TALL", raising=False)
    cfg, h, dev, ref = case(NAME)
    p = problem(cfg)
    assert moe.sizes(p)["tall_tile_m"] == 256, "the config must use the second tile list"
    return cfg, dev, p


def test_forward_graph_capture(gpu, monkeypatch):
    """Capture one moe_forward into a graph (after an eager call, which also
    creates the second stream) and replay it three times with other eager
    work on the stream between the replays: every replay writes the eager
    output's bits, and the buffer is cleared before each replay so a replay
    that skipped the forked launches could not pass on stale data."""
    cfg, dev, p = _setup(monkeypatch)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device="cuda")
    want = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    _forward(p, cfg, dev, want, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(want)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _forward(p, cfg, dev, out, ws)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    for i in range(3):
        out.zero_()
        ws.fill_(0x5A)                      # the workspace does not carry results over
        junk.normal_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {i} differs"
        assert float(junk.abs().sum()) > 0
    # and the eager call still agrees after the replays
    again = torch.empty_like(want)
    _forward(p, cfg, dev, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), want.view(torch.int16))


def test_forward_from_two_host_threads(gpu, monkeypatch):
    """Two host threads, each with its own stream, workspace and output,
    call moe_forward four times at once; each thread's results equal the
    single-threaded output bit for bit."""
    cfg, dev, p = _setup(monkeypatch)
    ws0 = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device="cuda")
    want = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    _forward(p, cfg, dev, want, ws0)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device="cuda")
            outs = [torch.empty_like(want) for _ in range(4)]
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for o in outs:
                    _forward(p, cfg, dev, o, ws)
            stream.synchronize()
            results[i] = outs
        except Exception as exc:           # reported in the main thread
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for i in range(2):
        for j, o in enumerate(results[i]):
            assert torch.equal(o.view(torch.int16), want.view(torch.int16)), f"thread {i} call {j}"
