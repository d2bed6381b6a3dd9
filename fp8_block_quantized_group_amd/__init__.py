"""Python binding of the gfx950 fp8 block-quantized MoE expert layer.

Argument marshalling only: every step runs in ``libmoe_fp8.so`` (HIP,
gfx950), declared in ``include/moe_fp8.h``.  PyTorch supplies device memory
and the current HIP stream.  Importing this package does not load the
library; the first call does, and raises if it is missing (build it with
``python -m fp8_block_quantized_group_amd.build``).  There is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_fp8.so")

Q_FP8_UE8M0, Q_FP8_F32, Q_BF16, Q_MXFP8 = 0, 1, 2, 3
W_FP8_BLOCK128, W_MXFP8, W_MXFP4 = 0, 1, 2
_ACT_QUANT = {"ue8m0": Q_FP8_UE8M0, "fp32": Q_FP8_F32, "bf16": Q_BF16, "mxfp8": Q_MXFP8}
_WEIGHT_QUANT = {"fp8_block128": W_FP8_BLOCK128, "mxfp8": W_MXFP8, "mxfp4": W_MXFP4}
ACTIVATIONS = ("silu", "gelu", "gelu_tanh", "silu_no_mul", "gelu_no_mul", "gelu_tanh_no_mul",
               "relu2_no_mul", "swigluoai", "swiglustep")   # moe_act_t order
LAYOUT_CONTIGUOUS, LAYOUT_BATCHED, LAYOUT_INDEXED = 0, 1, 2
_LAYOUT = {"contiguous": LAYOUT_CONTIGUOUS, "batched": LAYOUT_BATCHED, "indexed": LAYOUT_INDEXED}
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
           -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_LAUNCH"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "hidden", "intermediate", "num_experts", "top_k", "layout",
        "max_tokens_per_expert", "act_quant", "weight_quant", "activation")] + [
        ("act_limit", ctypes.c_float)]


class _Eplb(ctypes.Structure):
    _fields_ = [("logical_to_physical", ctypes.c_void_p), ("map_stride", ctypes.c_int32),
                ("replica_count", ctypes.c_void_p), ("num_logical", ctypes.c_int32),
                ("expert_load", ctypes.c_void_p), ("record_flag", ctypes.c_void_p),
                ("num_unpadded_tokens", ctypes.c_void_p)]


class _Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_num_tokens", "expert_offsets", "row_src", "slot_row", "tile_list")]


class _Sizes(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_int64), ("tile_list", ctypes.c_int64),
                ("stage_rows", ctypes.c_int64), ("expert_rows", ctypes.c_int64),
                ("x_sf_row", ctypes.c_int64), ("a2_sf_row", ctypes.c_int64),
                ("padded_rows", ctypes.c_int64), ("blocks", ctypes.c_int64),
                ("tile_m", ctypes.c_int32), ("tall_tile_m", ctypes.c_int32),
                ("max_tiles", ctypes.c_int64), ("tall_list_offset", ctypes.c_int64),
                ("max_tiles_tall", ctypes.c_int64)]


EXPORTS = ("moe_routing_sizes", "moe_stage_workspace_size", "moe_workspace_size",
           "moe_w2_workspace_size", "moe_stage",
           "moe_grouped_gemm_w13", "moe_grouped_gemm_w13_act", "moe_act_requant",
           "moe_grouped_gemm_w2", "moe_topk_reduce", "moe_align_capacity",
           "moe_align_block_size", "moe_grouped_gemm_w13_act_indexed",
           "moe_grouped_gemm_w2_indexed", "moe_fused_mul_sum", "moe_forward",
           "moe_forward_static", "moe_last_error")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m fp8_block_quantized_group_amd.build`")
    lib = ctypes.CDLL(path)
    P, V, S = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_routing_sizes.argtypes = [P(_Problem), P(_Sizes)]
    lib.moe_stage_workspace_size.argtypes = [P(_Problem), P(S)]
    lib.moe_workspace_size.argtypes = [P(_Problem), P(S)]
    lib.moe_w2_workspace_size.argtypes = [P(_Problem), P(S)]
    lib.moe_stage.argtypes = [P(_Problem), V, V, V, V, V, P(_Eplb), V, V, V, V, P(_Routing),
                              V, S, V]
    lib.moe_grouped_gemm_w13.argtypes = [P(_Problem), V, V, P(_Routing), V, V, V, V]
    lib.moe_grouped_gemm_w13_act.argtypes = [P(_Problem), V, V, P(_Routing), V, V, V, V, V]
    lib.moe_act_requant.argtypes = [P(_Problem), V, P(_Routing), V, V, V]
    lib.moe_grouped_gemm_w2.argtypes = [P(_Problem), V, V, P(_Routing), V, V, V, V, S, V]
    lib.moe_topk_reduce.argtypes = [P(_Problem), V, V, V, V, V]
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    lib.moe_align_capacity.argtypes = [P(_Problem), I32, P(I64), P(I64)]
    lib.moe_align_block_size.argtypes = [P(_Problem), V, P(_Routing), I32, V, V, V, V]
    lib.moe_grouped_gemm_w13_act_indexed.argtypes = [P(_Problem), V, V, V, V, V, I32, V, V, V,
                                                     V, V]
    lib.moe_grouped_gemm_w2_indexed.argtypes = [P(_Problem), V, V, V, V, V, I32, V, V, V, V,
                                                S, V]
    lib.moe_fused_mul_sum.argtypes = [P(_Problem), V, V, V, V, V]
    lib.moe_forward.argtypes = [P(_Problem), V, V, V, V, V, P(_Eplb), V, V, V, V, V, V, S, V]
    lib.moe_forward_static.argtypes = [P(_Problem), V, V, V, V, V, P(_Eplb), V, V, V, V, V, V]
    lib.moe_last_error.argtypes = []
    for name in EXPORTS:
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int if name != "moe_last_error" else ctypes.c_char_p
        # without argtypes ctypes passes Python ints as 32-bit C ints, which
        # would truncate every device pointer
        if fn.argtypes is None:
            raise RuntimeError(f"{name}: no ctypes signature declared")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, load_library().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclass(frozen=True)
class Problem:
    num_tokens: int
    hidden: int
    intermediate: int
    num_experts: int
    top_k: int
    layout: int = LAYOUT_CONTIGUOUS
    max_tokens_per_expert: int = 0
    act_quant: int = Q_FP8_UE8M0
    weight_quant: int = W_FP8_BLOCK128
    activation: int = 0                             # index into ACTIVATIONS
    act_limit: float = 0.0                          # clamp limit (moe_problem_t)

    def c(self) -> _Problem:
        return _Problem(self.num_tokens, self.hidden, self.intermediate, self.num_experts,
                        self.top_k, self.layout, self.max_tokens_per_expert, self.act_quant,
                        self.weight_quant, self.activation, self.act_limit)

    @staticmethod
    def from_config(cfg, act_quant: Optional[int] = None) -> "Problem":
        """From a ``moe_synth.MoeConfig``."""
        q = act_quant if act_quant is not None else _ACT_QUANT[cfg.act_quant]
        return Problem(cfg.T, cfg.K, cfg.N, cfg.E, cfg.top_k, _LAYOUT[cfg.layout],
                       cfg.max_tokens, q, _WEIGHT_QUANT[cfg.weight_quant],
                       ACTIVATIONS.index(cfg.activation), float(cfg.act_limit))


def sizes(p: Problem) -> dict:
    s = _Sizes()
    _check(load_library().moe_routing_sizes(ctypes.byref(p.c()), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in _Sizes._fields_}


def stage_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_stage_workspace_size(ctypes.byref(p.c()), ctypes.byref(n)))
    return n.value


def workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_workspace_size(ctypes.byref(p.c()), ctypes.byref(n)))
    return n.value


def w2_workspace_size(p: Problem) -> int:
    """Bytes of the w2 call's split-K workspace (0: w2 does not split)."""
    n = ctypes.c_size_t()
    _check(load_library().moe_w2_workspace_size(ctypes.byref(p.c()), ctypes.byref(n)))
    return n.value


def alloc_w2_workspace(p: Problem, device="cuda") -> Optional[torch.Tensor]:
    n = w2_workspace_size(p)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def _ws(ws: Optional[torch.Tensor]):
    return (_ptr(ws), ws.numel()) if ws is not None else (None, 0)


def _eplb(eplb: Optional[dict]):
    if eplb is None:
        return None
    l2p = eplb["l2p"]
    e = _Eplb(_ptr(l2p), l2p.shape[1], _ptr(eplb["replica_count"]), l2p.shape[0],
              _ptr(eplb.get("expert_load")), _ptr(eplb.get("record")),
              _ptr(eplb.get("num_unpadded")))
    return ctypes.byref(e), e


def _routing(r: dict) -> _Routing:
    return _Routing(*[_ptr(r[n]) for n in ("expert_num_tokens", "expert_offsets", "row_src",
                                          "slot_row", "tile_list")])


def scale_dtype(p: Problem):
    """torch dtype of the activation scales (E8M0 bytes or fp32)."""
    return torch.float32 if p.act_quant == Q_FP8_F32 else torch.uint8


def alloc_act_outputs(p: Problem, device="cuda", rows: Optional[int] = None):
    """(a2_q, a2_sf) for the w2 input: fp8 codes and scales, or bf16 values
    and None for unquantized activations; ``rows`` defaults to the layout's
    expert rows."""
    s = sizes(p)
    rows = s["expert_rows"] if rows is None else rows
    if p.act_quant == Q_BF16:
        return torch.empty((rows, p.intermediate), dtype=torch.bfloat16, device=device), None
    return (torch.empty((rows, p.intermediate), dtype=torch.uint8, device=device),
            torch.empty((rows, s["a2_sf_row"]), dtype=scale_dtype(p), device=device))


def alloc_stage_outputs(p: Problem, device="cuda") -> dict:
    """Caller-side buffers for moe_stage (allocated by torch)."""
    s = sizes(p)
    dev = torch.device(device)
    out = {
        "x_q": torch.empty((s["stage_rows"], p.hidden),
                           dtype=torch.bfloat16 if p.act_quant == Q_BF16 else torch.uint8,
                           device=dev),
        "x_sf": None if p.act_quant == Q_BF16 else torch.empty(
            (s["stage_rows"], s["x_sf_row"]), dtype=scale_dtype(p), device=dev),
        "topk_idx": torch.empty((p.num_tokens, p.top_k), dtype=torch.int64, device=dev),
        "topk_w": torch.empty((p.num_tokens, p.top_k), dtype=torch.float32, device=dev),
        "expert_num_tokens": torch.empty(p.num_experts, dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(p.num_experts + 1, dtype=torch.int32, device=dev),
        "row_src": torch.empty(max(s["slots"], 1), dtype=torch.int32, device=dev),
        "slot_row": torch.empty(max(s["slots"], 1), dtype=torch.int32, device=dev),
        "tile_list": torch.empty(s["tile_list"], dtype=torch.int32, device=dev),
        "ws": torch.empty(stage_workspace_size(p), dtype=torch.uint8, device=dev),
    }
    return out


def stage(p: Problem, hidden, topk_ids, topk_weights, bufs: dict, is_padding=None,
          expert_num_tokens=None, eplb=None):
    """moe_stage: fills bufs' x_q, x_sf, topk_idx, topk_w and the routing layout."""
    lib = load_library()
    e = _eplb(eplb)
    r = _routing(bufs)
    _check(lib.moe_stage(ctypes.byref(p.c()), _ptr(hidden), _ptr(expert_num_tokens),
                         _ptr(topk_ids), _ptr(topk_weights), _ptr(is_padding),
                         e[0] if e else None, _ptr(bufs["x_q"]), _ptr(bufs["x_sf"]),
                         _ptr(bufs["topk_idx"]), _ptr(bufs["topk_w"]), ctypes.byref(r),
                         _ptr(bufs["ws"]), bufs["ws"].numel(), _stream()))


def grouped_gemm_w13(p: Problem, a_q, a_sf, routing: dict, w13, w13_sf, gate_up):
    r = _routing(routing)
    _check(load_library().moe_grouped_gemm_w13(ctypes.byref(p.c()), _ptr(a_q), _ptr(a_sf),
                                                ctypes.byref(r), _ptr(w13), _ptr(w13_sf),
                                                _ptr(gate_up), _stream()))


def grouped_gemm_w13_act(p: Problem, a_q, a_sf, routing: dict, w13, w13_sf, a2_q, a2_sf):
    """w13 GEMM with SiLU(gate)*up and the fp8 re-quantization in its epilogue;
    a2_q / a2_sf equal grouped_gemm_w13 followed by act_requant bit for bit."""
    r = _routing(routing)
    _check(load_library().moe_grouped_gemm_w13_act(ctypes.byref(p.c()), _ptr(a_q), _ptr(a_sf),
                                                    ctypes.byref(r), _ptr(w13), _ptr(w13_sf),
                                                    _ptr(a2_q), _ptr(a2_sf), _stream()))


def act_requant(p: Problem, gate_up, routing: dict, a2_q, a2_sf):
    r = _routing(routing)
    _check(load_library().moe_act_requant(ctypes.byref(p.c()), _ptr(gate_up), ctypes.byref(r),
                                           _ptr(a2_q), _ptr(a2_sf), _stream()))


def grouped_gemm_w2(p: Problem, a2_q, a2_sf, routing: dict, w2, w2_sf, down, ws="auto"):
    """ws: the split-K workspace (alloc_w2_workspace); "auto" allocates it."""
    r = _routing(routing)
    if isinstance(ws, str):
        ws = alloc_w2_workspace(p, down.device)
    wp, wn = _ws(ws)
    _check(load_library().moe_grouped_gemm_w2(ctypes.byref(p.c()), _ptr(a2_q), _ptr(a2_sf),
                                               ctypes.byref(r), _ptr(w2), _ptr(w2_sf),
                                               _ptr(down), wp, wn, _stream()))


def topk_reduce(p: Problem, down, slot_row, topk_w, out):
    _check(load_library().moe_topk_reduce(ctypes.byref(p.c()), _ptr(down), _ptr(slot_row),
                                           _ptr(topk_w), _ptr(out), _stream()))


def align_capacity(p: Problem, block_size: int):
    """(sorted_ids length, expert_ids length) for ``block_size``."""
    n, b = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().moe_align_capacity(ctypes.byref(p.c()), block_size, ctypes.byref(n),
                                             ctypes.byref(b)))
    return n.value, b.value


def alloc_indexed(p: Problem, block_size: int, device="cuda") -> dict:
    """sorted_ids / expert_ids / num_tokens_padded buffers of the block map."""
    n, b = align_capacity(p, block_size)
    return {"sorted_ids": torch.empty(max(n, 1), dtype=torch.int32, device=device),
            "expert_ids": torch.empty(max(b, 1), dtype=torch.int32, device=device),
            "num_tokens_padded": torch.empty(1, dtype=torch.int32, device=device),
            "block_size": block_size}


def align_block_size(p: Problem, topk_idx, routing: dict, ix: dict):
    """moe_align_block_size: fills ix (from alloc_indexed) from moe_stage's
    topk_idx and routing."""
    r = _routing(routing)
    _check(load_library().moe_align_block_size(
        ctypes.byref(p.c()), _ptr(topk_idx), ctypes.byref(r), ix["block_size"],
        _ptr(ix["sorted_ids"]), _ptr(ix["expert_ids"]), _ptr(ix["num_tokens_padded"]),
        _stream()))


def grouped_gemm_w13_act_indexed(p: Problem, a_q, a_sf, ix: dict, w13, w13_sf, a2_q, a2_sf):
    _check(load_library().moe_grouped_gemm_w13_act_indexed(
        ctypes.byref(p.c()), _ptr(a_q), _ptr(a_sf), _ptr(ix["sorted_ids"]),
        _ptr(ix["expert_ids"]), _ptr(ix["num_tokens_padded"]), ix["block_size"], _ptr(w13),
        _ptr(w13_sf), _ptr(a2_q), _ptr(a2_sf), _stream()))


def grouped_gemm_w2_indexed(p: Problem, a2_q, a2_sf, ix: dict, w2, w2_sf, down, ws="auto"):
    if isinstance(ws, str):
        ws = alloc_w2_workspace(p, down.device)
    wp, wn = _ws(ws)
    _check(load_library().moe_grouped_gemm_w2_indexed(
        ctypes.byref(p.c()), _ptr(a2_q), _ptr(a2_sf), _ptr(ix["sorted_ids"]),
        _ptr(ix["expert_ids"]), _ptr(ix["num_tokens_padded"]), ix["block_size"], _ptr(w2),
        _ptr(w2_sf), _ptr(down), wp, wn, _stream()))


def fused_mul_sum(p: Problem, down, topk_idx, topk_w, out):
    _check(load_library().moe_fused_mul_sum(ctypes.byref(p.c()), _ptr(down), _ptr(topk_idx),
                                             _ptr(topk_w), _ptr(out), _stream()))


def forward(p: Problem, hidden, topk_ids, topk_weights, w13, w13_sf, w2, w2_sf, out, ws,
            is_padding=None, expert_num_tokens=None, eplb=None):
    """moe_forward: the whole layer; ``ws`` is a uint8 device tensor of at
    least workspace_size(p) bytes."""
    e = _eplb(eplb)
    _check(load_library().moe_forward(
        ctypes.byref(p.c()), _ptr(hidden), _ptr(expert_num_tokens), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(is_padding), e[0] if e else None, _ptr(w13), _ptr(w13_sf),
        _ptr(w2), _ptr(w2_sf), _ptr(out), _ptr(ws), ws.numel(), _stream()))


STATIC_SCRATCH_BYTES = 64 << 20      # MOE_STATIC_SCRATCH_BYTES


def forward_static(p: Problem, hidden, topk_ids, topk_weights, w13, w13_sf, w2, w2_sf, out,
                   is_padding=None, expert_num_tokens=None, eplb=None):
    """moe_forward_static: the whole layer with the library's static
    per-GPU workspace (no allocation; calls on one GPU must not overlap)."""
    e = _eplb(eplb)
    _check(load_library().moe_forward_static(
        ctypes.byref(p.c()), _ptr(hidden), _ptr(expert_num_tokens), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(is_padding), e[0] if e else None, _ptr(w13), _ptr(w13_sf),
        _ptr(w2), _ptr(w2_sf), _ptr(out), _stream()))


class MoeLayer:
    """The expert layer with its weights and a preallocated workspace."""

    def __init__(self, p: Problem, w13, w13_sf, w2, w2_sf):
        self.p = p
        self.w13, self.w13_sf, self.w2, self.w2_sf = w13, w13_sf, w2, w2_sf
        self.ws = torch.empty(workspace_size(p), dtype=torch.uint8, device=w13.device)

    def __call__(self, hidden, topk_ids, topk_weights, out=None, is_padding=None,
                 expert_num_tokens=None, eplb=None):
        if out is None:
            out = torch.empty((self.p.num_tokens, self.p.hidden), dtype=torch.bfloat16,
                              device=hidden.device)
        forward(self.p, hidden, topk_ids, topk_weights, self.w13, self.w13_sf, self.w2,
                self.w2_sf, out, self.ws, is_padding, expert_num_tokens, eplb)
        return out
