"""Python binding of libmoe_fp8 (block-scaled FP8 Mixture-of-Experts layer for MI355X / gfx950).

Argument marshalling only: every function checks devices, dtypes, shapes and contiguity, then
passes raw device pointers and the current HIP stream to the C ABI declared in
``include/moe_fp8.h``.  All computation happens in the HIP kernels; there is no fallback.  If the
library has not been built, importing works but the first call raises ``MoeLibraryMissing``
(build with ``python -m block_scaled_fp8_top_amd.build``).

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")

MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ARG, MOE_ERR_HIP, MOE_ERR_WORKSPACE = -1, -2, -3, -4, -5, -6
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_EPI_STORE, MOE_EPI_SWIGLU_QUANT = 0, 1
MOE_OP_DISPATCH, MOE_OP_GROUPED_GEMM = 1, 2
MOE_B_ROWMAJOR, MOE_B_PACKED, MOE_B_PACKED_FP4 = 0, 1, 2
MOE_SCALE_AMAX, MOE_SCALE_POW2 = 0, 1

EXPORTED = ("moe_gate_logits", "moe_route", "moe_route_quant", "moe_replay_route", "moe_replay_gate", "moe_router_score_eval",
            "moe_quant_fp8_block",
            "moe_dispatch", "moe_dispatch_plan", "moe_pack_weights_fp8", "moe_packed_weight_bytes", "moe_grouped_gemm_plan",
            "moe_grouped_gemm_fp8_planned", "moe_grouped_gemm_fp8_swiglu_save", "moe_grouped_gemm_fp8_gather",
            "moe_grouped_gemm_fp8", "moe_grouped_gemm_fp8_noalloc", "moe_combine", "moe_combine_residual", "moe_payload_bytes",
            "moe_payload_pack", "moe_payload_unpack", "moe_payload_to_host", "moe_payload_from_host",
            "moe_combine_backward", "moe_swiglu_backward_quant", "moe_route_backward", "moe_gate_backward",
            "moe_gate_backward_workspace", "moe_transpose_fp8_blocks", "moe_wgrad_max_tiles", "moe_wgrad_tiles",
            "moe_colwise_quant_rows", "moe_colwise_quant_swiglu", "moe_grouped_gemm_wgrad", "moe_quant_mxfp4",
            "moe_packed_fp4_bytes", "moe_pack_weights_fp4",
            "moe_workspace_bytes", "moe_status_str", "moe_version")


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: status {code} ({status_str(code)})")
        self.code = code


class GemmPlan(ctypes.Structure):
    """Host half of a grouped-GEMM tile plan (the tile list itself lives in the workspace)."""
    _fields_ = [("tile_rows", ctypes.c_int32), ("groups", ctypes.c_int32), ("max_rows", ctypes.c_int64),
                ("workspace", ctypes.c_void_p)]


class RouterCfg(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("group_score_topk", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded shared library (raises MoeLibraryMissing if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeLibraryMissing(f"{LIB_PATH} not found; build it with `python -m block_scaled_fp8_top_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(RouterCfg)
    sig = {
        "moe_gate_logits": [P, ctypes.c_int, P, P, I64, I32, I32, P, P],
        "moe_route": [P, I64, cfgp, P, P, P, I64, P],
        "moe_replay_route": [P, I64, cfgp, P, I64, P, P, P, P],
        "moe_replay_gate": [P, ctypes.c_int, P, P, I64, I32, cfgp, P, I64, P, P, P, P],
        "moe_router_score_eval": [P, I64, ctypes.c_int, P, P],
        "moe_quant_fp8_block": [P, ctypes.c_int, I64, I64, I32, I32, I32, P, P, P],
        "moe_route_quant": [P, I64, ctypes.POINTER(RouterCfg), P, P, P, I64, P, ctypes.c_int, I32, I32, P, P, P],
        "moe_dispatch": [P, I64, I32, I32, I32, P, P, I32, P, P, P, P, P, P, P, SZ, P],
        "moe_dispatch_plan": [P, I64, I32, I32, I32, P, P, I32, P, P, P, P, P, P, P, SZ, I32, P, SZ,
                              ctypes.POINTER(GemmPlan), P],
        "moe_pack_weights_fp8": [P, I32, I32, I32, I32, P, P],
        "moe_packed_weight_bytes": [I32, I32, I32, I32],
        "moe_grouped_gemm_fp8": [P, P, P, I32, I64, P, I32, P, I32, I32, I32, I32, I32, P, ctypes.c_int, P, P, SZ, P],
        "moe_grouped_gemm_fp8_noalloc": [P, P, P, I32, I64, P, I32, P, I32, I32, I32, I32, I32, P, ctypes.c_int, P, P],
        "moe_grouped_gemm_plan": [P, I32, I64, I32, P, SZ, ctypes.POINTER(GemmPlan), P],
        "moe_grouped_gemm_fp8_planned": [ctypes.POINTER(GemmPlan), P, P, P, P, I32, P, I32, I32, I32, I32, P,
                                         ctypes.c_int, P, P],
        "moe_grouped_gemm_fp8_swiglu_save": [ctypes.POINTER(GemmPlan), P, P, P, P, I32, P, I32, I32, I32, P, P, P,
                                             P],
        "moe_grouped_gemm_fp8_gather": [ctypes.POINTER(GemmPlan), P, I64, P, P, P, P, I32, P, I32, I32, I32, I32, P,
                                        ctypes.c_int, P, P, P],
        "moe_combine": [P, ctypes.c_int, P, P, I64, I32, I32, P, P, ctypes.c_int, P],
        "moe_combine_residual": [P, ctypes.c_int, P, P, I64, I32, I32, P, P, P, P, ctypes.c_int, P],
        "moe_payload_bytes": [I64, I32],
        "moe_payload_pack": [P, I64, I32, P, P, P],
        "moe_payload_unpack": [P, I64, I32, P, P],
        "moe_payload_to_host": [P, I64, I32, P, P, P, P],
        "moe_payload_from_host": [P, I64, I32, P, P, P],
        "moe_combine_backward": [P, ctypes.c_int, P, ctypes.c_int, P, P, I64, I32, I32, P, I32, P, P, P, P, P],
        "moe_wgrad_max_tiles": [I64, I32],
        "moe_quant_mxfp4": [P, ctypes.c_int, I64, I32, P, P, P],
        "moe_packed_fp4_bytes": [I32, I32, I32, I32, P],
        "moe_pack_weights_fp4": [P, P, I32, I32, I32, I32, P, P, P],
        "moe_wgrad_tiles": [P, I32, P, P],
        "moe_colwise_quant_rows": [P, ctypes.c_int, P, P, P, P, I32, I64, I32, I32, P, P, P],
        "moe_colwise_quant_swiglu": [P, P, I32, P, P, I32, I64, I32, P, P, P],
        "moe_grouped_gemm_wgrad": [P, P, I32, P, P, I32, P, I32, I64, I32, P, P],
        "moe_swiglu_backward_quant": [P, P, I64, I32, I32, P, P, P],
        "moe_route_backward": [P, P, P, I64, cfgp, P, P],
        "moe_gate_backward": [P, P, ctypes.c_int, P, I64, I32, I32, P, P, ctypes.c_int, P, P, P, SZ, P],
        "moe_gate_backward_workspace": [I64, I32, I32],
        "moe_transpose_fp8_blocks": [P, P, I32, I32, I32, P, P, P],
        "moe_workspace_bytes": [ctypes.c_int, I64, I32, I32, I32, I32],
        "moe_status_str": [ctypes.c_int],
        "moe_version": [],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.moe_workspace_bytes.restype = ctypes.c_size_t
    L.moe_packed_weight_bytes.restype = ctypes.c_size_t
    L.moe_payload_bytes.restype = ctypes.c_size_t
    L.moe_gate_backward_workspace.restype = ctypes.c_size_t
    L.moe_wgrad_max_tiles.restype = ctypes.c_int64
    L.moe_packed_fp4_bytes.restype = ctypes.c_size_t
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_version.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().moe_status_str(int(code)).decode()


def version() -> str:
    return lib().moe_version().decode()


def workspace_bytes(op: int, rows_or_T: int, k: int, E: int, N: int = 0, K: int = 0) -> int:
    return int(lib().moe_workspace_bytes(op, rows_or_T, k, E, N, K))


# ----------------------------------------------------------------------------- marshalling helpers
def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _act_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activation dtype {t.dtype} unsupported (float32 or bfloat16)")


def _check(code: int, what: str):
    if code != MOE_OK:
        raise MoeError(code, what)


FP8 = torch.uint8  # e4m3 codes are carried as raw bytes


def router_cfg(num_experts, top_k, score_fn, renormalize, n_group=1, topk_group=1, group_score_topk=2) -> RouterCfg:
    sf = score_fn if isinstance(score_fn, int) else (MOE_SCORE_SOFTMAX if score_fn == "softmax" else MOE_SCORE_SIGMOID)
    return RouterCfg(num_experts, top_k, sf, int(bool(renormalize)), n_group, topk_group, group_score_topk)


# ----------------------------------------------------------------------------- the seven calls
def moe_gate_logits(x: torch.Tensor, wg: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, H = x.shape
    E = wg.shape[0]
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(wg, "wg", torch.float32, (E, H))
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    out = torch.empty((T, E), dtype=torch.float32, device=x.device) if out is None else _dev(out, "out", torch.float32, (T, E))
    _check(lib().moe_gate_logits(_p(x), _act_code(x), _p(wg), _p(bias), T, H, E, _p(out), _stream(stream)),
           "moe_gate_logits")
    return out


def moe_route(logits: torch.Tensor, cfg: RouterCfg, record: Optional[torch.Tensor] = None, topk_idx=None,
              topk_w=None, stream=None):
    """Returns (topk_idx [T,k] int32, topk_w [T,k] fp32).  ``record`` is one layer of the routing
    payload, an int32 [k, seq_len>=T] view (contiguous rows)."""
    T, E = logits.shape
    _dev(logits, "logits", torch.float32)
    if E != cfg.num_experts:
        raise ValueError("logits width != num_experts")
    k = cfg.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device) if topk_idx is None else _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if topk_w is None else _dev(topk_w, "topk_w", torch.float32, (T, k))
    rec_ptr, rec_ld = None, 0
    if record is not None:
        if record.device.type != "cuda" or record.dtype != torch.int32 or record.dim() != 2 or record.shape[0] != k \
                or record.stride(1) != 1:
            raise ValueError("record must be a cuda int32 [k, seq_len] view with unit column stride")
        rec_ptr, rec_ld = _p(record), record.stride(0)
        if record.shape[1] < T:
            raise ValueError("record seq_len < T")
    _check(lib().moe_route(_p(logits), T, ctypes.byref(cfg), _p(idx), _p(w), rec_ptr, rec_ld, _stream(stream)),
           "moe_route")
    return idx, w


def moe_route_quant(logits: torch.Tensor, cfg: RouterCfg, x: torch.Tensor, record: Optional[torch.Tensor] = None,
                    topk_idx=None, topk_w=None, q=None, scales=None, stream=None, pow2: bool = False):
    """moe_route and the 1x128 quantisation of x [T,H] in one launch; returns (topk_idx, topk_w, q, scales)."""
    T, E = logits.shape
    _dev(logits, "logits", torch.float32)
    _dev(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() != 2 or x.shape[0] != T or x.shape[1] % 128:
        raise ValueError("x must be [T, H] with H % 128 == 0")
    H = x.shape[1]
    if E != cfg.num_experts:
        raise ValueError("logits width != num_experts")
    k = cfg.top_k
    dev = logits.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else _dev(topk_w, "topk_w", torch.float32, (T, k))
    q = torch.empty((T, H), dtype=FP8, device=dev) if q is None else _dev(q, "q", FP8, (T, H))
    scales = torch.empty((T, H // 128), dtype=torch.float32, device=dev) if scales is None else \
        _dev(scales, "scales", torch.float32, (T, H // 128))
    rec_ptr, rec_ld = None, 0
    if record is not None:
        if record.device.type != "cuda" or record.dtype != torch.int32 or record.dim() != 2 or record.shape[0] != k \
                or record.stride(1) != 1 or record.shape[1] < T:
            raise ValueError("record must be a cuda int32 [k, seq_len>=T] view with unit column stride")
        rec_ptr, rec_ld = _p(record), record.stride(0)
    _check(lib().moe_route_quant(_p(logits), T, ctypes.byref(cfg), _p(idx), _p(w), rec_ptr, rec_ld, _p(x), _act_code(x),
                                 H, MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX, _p(q), _p(scales), _stream(stream)),
           "moe_route_quant")
    return idx, w, q, scales


def moe_replay_route(logits: torch.Tensor, cfg: RouterCfg, replay: torch.Tensor, bad_count: Optional[torch.Tensor] = None,
                     topk_idx=None, topk_w=None, stream=None):
    """Returns (topk_idx, topk_w).  ``replay``: int32 [k, seq_len>=T] view of one payload layer;
    ``bad_count``: optional cuda int32 [1] accumulator of rejected tokens."""
    T, E = logits.shape
    _dev(logits, "logits", torch.float32)
    k = cfg.top_k
    if replay.device.type != "cuda" or replay.dtype != torch.int32 or replay.dim() != 2 or replay.shape[0] != k \
            or replay.stride(1) != 1 or replay.shape[1] < T:
        raise ValueError("replay must be a cuda int32 [k, seq_len>=T] view with unit column stride")
    if bad_count is not None:
        _dev(bad_count, "bad_count", torch.int32, (1,))
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device) if topk_idx is None else _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if topk_w is None else _dev(topk_w, "topk_w", torch.float32, (T, k))
    _check(lib().moe_replay_route(_p(logits), T, ctypes.byref(cfg), _p(replay), replay.stride(0), _p(idx), _p(w),
                                  _p(bad_count), _stream(stream)), "moe_replay_route")
    return idx, w


def moe_replay_gate(x: torch.Tensor, wg: torch.Tensor, bias: Optional[torch.Tensor], cfg: RouterCfg,
                    replay: torch.Tensor, bad_count: Optional[torch.Tensor] = None, topk_idx=None, topk_w=None,
                    stream=None):
    """Sigmoid routers: replay fused with the gate projection (only the k recorded logits per
    token).  Same (topk_idx, topk_w) as moe_gate_logits + moe_replay_route, bit for bit."""
    T, H = x.shape
    E = wg.shape[0]
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(wg, "wg", torch.float32, (E, H))
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    k = cfg.top_k
    if replay.device.type != "cuda" or replay.dtype != torch.int32 or replay.dim() != 2 or replay.shape[0] != k \
            or replay.stride(1) != 1 or replay.shape[1] < T:
        raise ValueError("replay must be a cuda int32 [k, seq_len>=T] view with unit column stride")
    if bad_count is not None:
        _dev(bad_count, "bad_count", torch.int32, (1,))
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if topk_idx is None else _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    w = torch.empty((T, k), dtype=torch.float32, device=x.device) if topk_w is None else _dev(topk_w, "topk_w", torch.float32, (T, k))
    code = MOE_BF16 if x.dtype == torch.bfloat16 else MOE_F32
    _check(lib().moe_replay_gate(_p(x), code, _p(wg), _p(bias), T, H, ctypes.byref(cfg), _p(replay), replay.stride(0),
                                 _p(idx), _p(w), _p(bad_count), _stream(stream)), "moe_replay_gate")
    return idx, w


def moe_router_score_eval(x: torch.Tensor, score_fn, out=None, stream=None) -> torch.Tensor:
    """The router's fixed exp (score_fn softmax) or sigmoid, elementwise on fp32 x."""
    _dev(x, "x", torch.float32)
    sf = score_fn if isinstance(score_fn, int) else (MOE_SCORE_SOFTMAX if score_fn == "softmax" else MOE_SCORE_SIGMOID)
    out = torch.empty_like(x) if out is None else _dev(out, "out", torch.float32, x.shape)
    _check(lib().moe_router_score_eval(_p(x), x.numel(), sf, _p(out), _stream(stream)), "moe_router_score_eval")
    return out


def moe_quant_fp8_block(x: torch.Tensor, block_rows: int, q=None, scales=None, stream=None, pow2: bool = False):
    """x: [rows, cols] or [batch, rows, cols] fp32/bf16 -> (codes uint8 same shape, scales fp32);
    pow2: power-of-two scales (the form the GEMM applies in the matrix cores)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    xx = x if x.dim() == 3 else x.unsqueeze(0)
    B, R, C = xx.shape
    if block_rows not in (1, 128) or C % 128 or R % block_rows:
        raise ValueError("cols must be a multiple of 128 and rows a multiple of block_rows (1 or 128)")
    sshape = (B, R // block_rows, C // 128) if x.dim() == 3 else (R // block_rows, C // 128)
    q = torch.empty(x.shape, dtype=FP8, device=x.device) if q is None else _dev(q, "q", FP8, x.shape)
    scales = torch.empty(sshape, dtype=torch.float32, device=x.device) if scales is None else _dev(scales, "scales", torch.float32, sshape)
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_quant_fp8_block(_p(x), _act_code(x), B, R, C, block_rows, mode, _p(q), _p(scales),
                                     _stream(stream)), "moe_quant_fp8_block")
    return q, scales


@dataclass
class Dispatched:
    counts: torch.Tensor      # [G] int32
    offsets: torch.Tensor     # [G+1] int32
    dest_row: torch.Tensor    # [T,k] int32
    src_token: torch.Tensor   # [max_rows] int32
    aq: Optional[torch.Tensor]   # [max_rows, H] uint8 (rows beyond offsets[G] unwritten)
    as_: Optional[torch.Tensor]  # [max_rows, H/128] fp32
    max_rows: int


def _check_dispatched(out: Dispatched, T: int, k: int, G: int, max_rows: int, H: int):
    """Caller-provided dispatch outputs: the kernels write exactly these extents."""
    _dev(out.counts, "counts", torch.int32, (G,))
    _dev(out.offsets, "offsets", torch.int32, (G + 1,))
    _dev(out.dest_row, "dest_row", torch.int32, (T, k))
    _dev(out.src_token, "src_token", torch.int32)
    if out.src_token.numel() < max_rows:
        raise ValueError("src_token holds fewer than T*k (+T) rows")
    if out.aq is not None:
        _dev(out.aq, "aq", FP8, (max_rows, H))
    if out.as_ is not None:
        _dev(out.as_, "as", torch.float32, (max_rows, H // 128))


def moe_dispatch(topk_idx: torch.Tensor, num_experts: int, append_shared: bool, xq: Optional[torch.Tensor] = None,
                 xs: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 out: Optional[Dispatched] = None, stream=None, copy_codes: bool = True) -> Dispatched:
    """copy_codes=False: only the scales are permuted (aq is None); the grouped GEMM then gathers
    the codes from xq through src_token (moe_grouped_gemm_fp8 with a_rows)."""
    T, k = topk_idx.shape
    _dev(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    G = num_experts + (1 if append_shared else 0)
    max_rows = T * k + (T if append_shared else 0)
    H = 0
    if xq is not None:
        H = xq.shape[1]
        _dev(xq, "xq", FP8, (T, H))
        _dev(xs, "xs", torch.float32, (T, H // 128))
    ws_need = workspace_bytes(MOE_OP_DISPATCH, T, k, num_experts)
    if workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    elif _dev(workspace, "workspace", torch.uint8).numel() < ws_need:
        raise ValueError("workspace too small")
    if out is None:
        out = Dispatched(
            counts=torch.empty(G, dtype=torch.int32, device=dev),
            offsets=torch.empty(G + 1, dtype=torch.int32, device=dev),
            dest_row=torch.empty((T, k), dtype=torch.int32, device=dev),
            src_token=torch.empty(max(max_rows, 1), dtype=torch.int32, device=dev),
            aq=torch.empty((max_rows, H), dtype=FP8, device=dev) if xq is not None and copy_codes else None,
            as_=torch.empty((max_rows, H // 128), dtype=torch.float32, device=dev) if xq is not None else None,
            max_rows=max_rows)
    else:
        _check_dispatched(out, T, k, G, max_rows, H)
    _check(lib().moe_dispatch(_p(topk_idx), T, k, num_experts, int(bool(append_shared)), _p(xq), _p(xs), H,
                              _p(out.counts), _p(out.offsets), _p(out.dest_row), _p(out.src_token), _p(out.aq),
                              _p(out.as_), _p(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "moe_dispatch")
    return out


def moe_dispatch_plan(topk_idx: torch.Tensor, num_experts: int, append_shared: bool, xq: Optional[torch.Tensor],
                      xs: Optional[torch.Tensor], workspace: torch.Tensor, out: Dispatched, gemm_workspace: torch.Tensor,
                      tile_rows: int = 0, stream=None):
    """moe_dispatch into ``out`` followed by the grouped GEMM's tile plan of its groups (held in
    ``gemm_workspace``); for one-workgroup batches the dispatch kernel writes the plan itself.
    Returns the GemmPlan to pass as ``plan=`` to moe_grouped_gemm_fp8."""
    T, k = topk_idx.shape
    _dev(topk_idx, "topk_idx", torch.int32)
    H = 0
    if xq is not None:
        H = xq.shape[1]
        _dev(xq, "xq", FP8, (T, H))
        _dev(xs, "xs", torch.float32, (T, H // 128))
    _check_dispatched(out, T, k, num_experts + (1 if append_shared else 0), T * k + (T if append_shared else 0), H)
    _dev(workspace, "workspace", torch.uint8)
    _dev(gemm_workspace, "gemm_workspace", torch.uint8)
    if workspace.numel() * workspace.element_size() < workspace_bytes(MOE_OP_DISPATCH, T, k, num_experts):
        raise ValueError("workspace too small")
    plan = GemmPlan()
    _check(lib().moe_dispatch_plan(_p(topk_idx), T, k, num_experts, int(bool(append_shared)), _p(xq), _p(xs), H,
                                   _p(out.counts), _p(out.offsets), _p(out.dest_row), _p(out.src_token), _p(out.aq),
                                   _p(out.as_), _p(workspace), workspace.numel() * workspace.element_size(),
                                   tile_rows, _p(gemm_workspace), gemm_workspace.numel() * gemm_workspace.element_size(),
                                   ctypes.byref(plan), _stream(stream)), "moe_dispatch_plan")
    plan._keep = gemm_workspace
    return plan


def packed_weight_bytes(groups: int, N: int, K: int, epilogue: int) -> int:
    return int(lib().moe_packed_weight_bytes(groups, N, K, epilogue))


@dataclass
class PackedWeight:
    """A [G,N,K] e4m3 weight rearranged by moe_pack_weights_fp8 for one GEMM epilogue."""
    data: torch.Tensor   # [G, packed bytes per group] uint8
    G: int
    N: int
    K: int
    epilogue: int


def moe_pack_weights_fp8(b: torch.Tensor, epilogue: int, out: Optional[torch.Tensor] = None, stream=None) -> PackedWeight:
    """b [G,N,K] e4m3 bytes (device) -> the packed layout the grouped GEMM streams for ``epilogue``."""
    _dev(b, "b", FP8)
    G, N, K = b.shape
    nbytes = packed_weight_bytes(G, N, K, epilogue)
    if nbytes == 0:
        raise MoeError(MOE_ERR_SHAPE, f"moe_pack_weights_fp8: unsupported shape {tuple(b.shape)} / epilogue {epilogue}")
    if out is None:
        out = torch.empty((G, nbytes // G), dtype=torch.uint8, device=b.device)
    else:
        _dev(out, "out", torch.uint8, (G, nbytes // G))
    _check(lib().moe_pack_weights_fp8(_p(b), G, N, K, epilogue, _p(out), _stream(stream)), "moe_pack_weights_fp8")
    return PackedWeight(out, G, N, K, epilogue)


@dataclass
class PackedWeightFP4:
    """A [G,N,K] FP4 weight (two codes per byte) with its E8M0 scales, packed by
    moe_pack_weights_fp4 for one GEMM epilogue."""
    data: torch.Tensor     # [G, code bytes per group] uint8
    scales: torch.Tensor   # [G, scale-image bytes per group] uint8
    G: int
    N: int
    K: int
    epilogue: int


def moe_quant_mxfp4(w: torch.Tensor, q=None, e8=None, stream=None):
    """w [..., rows, cols] fp32/bf16 -> (codes [..., rows, cols/2] uint8, E8M0 scale codes
    [..., rows, cols/32] uint8): FP4 E2M1 in 1x32 blocks with power-of-two scales."""
    _dev(w, "w", (torch.float32, torch.bfloat16))
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    qs, es = tuple(w.shape[:-1]) + (cols // 2,), tuple(w.shape[:-1]) + (cols // 32,)
    q = torch.empty(qs, dtype=torch.uint8, device=w.device) if q is None else _dev(q, "q", torch.uint8, qs)
    e8 = torch.empty(es, dtype=torch.uint8, device=w.device) if e8 is None else _dev(e8, "e8", torch.uint8, es)
    _check(lib().moe_quant_mxfp4(_p(w), _act_code(w), rows, cols, _p(q), _p(e8), _stream(stream)), "moe_quant_mxfp4")
    return q, e8


def moe_pack_weights_fp4(q: torch.Tensor, e8: torch.Tensor, epilogue: int, stream=None) -> PackedWeightFP4:
    """q [G,N,K/2], e8 [G,N,K/32] (from moe_quant_mxfp4) -> the packed FP4 layout of ``epilogue``."""
    _dev(q, "q", torch.uint8)
    G, N, K2 = q.shape
    K = 2 * K2
    _dev(e8, "e8", torch.uint8, (G, N, K // 32))
    sb = ctypes.c_size_t(0)
    nbytes = int(lib().moe_packed_fp4_bytes(G, N, K, epilogue, ctypes.byref(sb)))
    if nbytes == 0:
        raise MoeError(MOE_ERR_SHAPE, f"moe_pack_weights_fp4: unsupported shape {(G, N, K)} / epilogue {epilogue}")
    data = torch.empty((G, nbytes // G), dtype=torch.uint8, device=q.device)
    scales = torch.empty((G, sb.value // G), dtype=torch.uint8, device=q.device)
    _check(lib().moe_pack_weights_fp4(_p(q), _p(e8), G, N, K, epilogue, _p(data), _p(scales), _stream(stream)),
           "moe_pack_weights_fp4")
    return PackedWeightFP4(data, scales, G, N, K, epilogue)


def moe_grouped_gemm_plan(offsets: torch.Tensor, max_rows: int, workspace: torch.Tensor, tile_rows: int = 0,
                          stream=None):
    """Tile plan of the groups in ``offsets`` [G+1] (device) for up to max_rows rows, written into
    ``workspace``; returns the host plan to pass as ``plan=`` to moe_grouped_gemm_fp8.  The
    workspace must not be reused until the GEMMs that use the plan have run."""
    G = offsets.shape[0] - 1
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    plan = GemmPlan()
    _check(lib().moe_grouped_gemm_plan(_p(offsets), G, max_rows, tile_rows, _p(workspace),
                                       workspace.numel() * workspace.element_size(), ctypes.byref(plan),
                                       _stream(stream)), "moe_grouped_gemm_plan")
    plan._keep = workspace   # the tile list lives there
    return plan


def moe_grouped_gemm_fp8(a: torch.Tensor, as_: torch.Tensor, offsets: torch.Tensor, b, bs: torch.Tensor,
                         epilogue: int = MOE_EPI_STORE, out_dtype=torch.bfloat16, out=None, out_scales=None,
                         workspace: Optional[torch.Tensor] = None, stream=None, tile_rows: int = 0,
                         plan: Optional[GemmPlan] = None, pow2: bool = False, save_g: Optional[torch.Tensor] = None,
                         a_rows: Optional[torch.Tensor] = None):
    """a [max_rows,K] uint8, as_ [max_rows,K/128], offsets [G+1] (device), b [G,N,K] uint8 or a
    PackedWeight packed for this epilogue, bs [G,N/128,K/128].
    STORE -> out [max_rows,N] (bf16/fp32); SWIGLU_QUANT -> (h codes [max_rows,N/2] uint8, scales [max_rows,N/256]).
    tile_rows: 32, 48, 64, 128 or 256 (packed weights only) rows per workgroup tile, 0 = chosen from
    the group sizes.
    plan: a plan from moe_grouped_gemm_plan for these offsets and max_rows (then no workspace is
    needed and tile_rows is the plan's).  pow2: every scale in as_ and bs is a power of two (the
    matrix cores apply them; the SwiGLU epilogue writes power-of-two scales for h).
    save_g (SwiGLU with a plan only): fp32 [max_rows, N] that also receives the GEMM output G.
    a_rows (with a plan only): int32 [max_rows] (the dispatch's src_token); group row r then reads
    the codes of row a_rows[r] of a [a_count, K], while as_ [max_rows, K/128] stays in group order."""
    a_count, K = a.shape
    max_rows = as_.shape[0] if a_rows is not None else a_count
    if isinstance(b, PackedWeightFP4):
        if b.epilogue != epilogue:
            raise ValueError("weight was packed for another epilogue")
        if not pow2:
            raise ValueError("FP4 weights need power-of-two activation scales (pow2=True)")
        G, N, Kb, b_layout, b_t = b.G, b.N, b.K, MOE_B_PACKED_FP4, b.data
        bs = b.scales
    elif isinstance(b, PackedWeight):
        if b.epilogue != epilogue:
            raise ValueError("weight was packed for another epilogue")
        G, N, Kb, b_layout, b_t = b.G, b.N, b.K, MOE_B_PACKED, b.data
        _dev(b_t, "b", torch.uint8, (G, packed_weight_bytes(G, N, Kb, epilogue) // G))
    else:
        G, N, Kb = b.shape
        b_layout, b_t = MOE_B_ROWMAJOR, b
        _dev(b, "b", FP8)
    if Kb != K:
        raise ValueError("K mismatch")
    _dev(a, "a", FP8)
    _dev(as_, "as", torch.float32, (max_rows, K // 128))
    if a_rows is not None:
        _dev(a_rows, "a_rows", torch.int32)
        if a_rows.shape[0] < max_rows or plan is None:
            raise ValueError("a_rows needs a plan and one entry per group row")
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    if b_layout == MOE_B_PACKED_FP4:
        _dev(bs, "bs", torch.uint8)
    else:
        _dev(bs, "bs", torch.float32, (G, N // 128, K // 128))
    dev = a.device
    if plan is not None:
        if plan.groups != G or plan.max_rows != max_rows:
            raise ValueError("plan was made for other groups / rows")
    else:
        ws_need = workspace_bytes(MOE_OP_GROUPED_GEMM, max_rows, 0, G, N, K)
        if workspace is None:
            workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        elif workspace.numel() * workspace.element_size() < ws_need:
            raise ValueError("workspace too small")
    if epilogue == MOE_EPI_STORE:
        code = MOE_BF16 if out_dtype == torch.bfloat16 else MOE_F32
        out = torch.empty((max_rows, N), dtype=out_dtype, device=dev) if out is None else _dev(out, "out", out_dtype, (max_rows, N))
        osc = None
    else:
        code = MOE_FP8_E4M3
        F = N // 2
        out = torch.empty((max_rows, F), dtype=FP8, device=dev) if out is None else _dev(out, "out", FP8, (max_rows, F))
        osc = torch.empty((max_rows, F // 128), dtype=torch.float32, device=dev) if out_scales is None else \
            _dev(out_scales, "out_scales", torch.float32, (max_rows, F // 128))
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    if save_g is not None and (plan is None or epilogue != MOE_EPI_SWIGLU_QUANT):
        raise ValueError("save_g needs a plan and the SwiGLU epilogue")
    if save_g is not None:
        _dev(save_g, "save_g", torch.float32, (max_rows, N))
    if a_rows is not None:
        _check(lib().moe_grouped_gemm_fp8_gather(ctypes.byref(plan), _p(a), a_count, _p(a_rows), _p(as_), _p(offsets),
                                                 _p(b_t), b_layout, _p(bs), N, K, epilogue, mode, _p(out), code,
                                                 _p(osc), _p(save_g), _stream(stream)), "moe_grouped_gemm_fp8_gather")
        return out if epilogue == MOE_EPI_STORE else (out, osc)
    if save_g is not None:
        _check(lib().moe_grouped_gemm_fp8_swiglu_save(ctypes.byref(plan), _p(a), _p(as_), _p(offsets), _p(b_t),
                                                      b_layout, _p(bs), N, K, mode, _p(out), _p(osc), _p(save_g),
                                                      _stream(stream)), "moe_grouped_gemm_fp8_swiglu_save")
        return out, osc
    if plan is not None:
        _check(lib().moe_grouped_gemm_fp8_planned(ctypes.byref(plan), _p(a), _p(as_), _p(offsets), _p(b_t), b_layout,
                                                  _p(bs), N, K, epilogue, mode, _p(out), code, _p(osc),
                                                  _stream(stream)),
               "moe_grouped_gemm_fp8_planned")
        return out if epilogue == MOE_EPI_STORE else (out, osc)
    _check(lib().moe_grouped_gemm_fp8(_p(a), _p(as_), _p(offsets), G, max_rows, _p(b_t), b_layout, _p(bs), N, K,
                                      epilogue, mode, tile_rows, _p(out),
                                      code, _p(osc), _p(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "moe_grouped_gemm_fp8")
    return out if epilogue == MOE_EPI_STORE else (out, osc)


NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_grouped_gemm_fp8_noalloc(a: torch.Tensor, as_: torch.Tensor, offsets: torch.Tensor, b, bs: torch.Tensor,
                                 epilogue: int, out: torch.Tensor, out_scales: Optional[torch.Tensor] = None,
                                 tile_rows: int = 0, pow2: bool = False, stream=None):
    """moe_grouped_gemm_fp8 with the tile plan in the library's own device scratch (no workspace,
    nothing allocated here either): ``out`` (and ``out_scales`` for the SwiGLU epilogue) must be given.
    Results are bitwise those of moe_grouped_gemm_fp8."""
    max_rows, K = a.shape
    if isinstance(b, PackedWeight):
        if b.epilogue != epilogue:
            raise ValueError("weight was packed for another epilogue")
        G, N, Kb, b_layout, b_t = b.G, b.N, b.K, MOE_B_PACKED, b.data
    elif isinstance(b, PackedWeightFP4):
        G, N, Kb, b_layout, b_t = b.G, b.N, b.K, MOE_B_PACKED_FP4, b.data
        bs = b.scales
    else:
        G, N, Kb = b.shape
        b_layout, b_t = MOE_B_ROWMAJOR, _dev(b, "b", FP8)
    if Kb != K:
        raise ValueError("K mismatch")
    _dev(a, "a", FP8)
    _dev(as_, "as", torch.float32, (max_rows, K // 128))
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    if epilogue == MOE_EPI_STORE:
        _dev(out, "out", (torch.float32, torch.bfloat16), (max_rows, N))
        code = MOE_BF16 if out.dtype == torch.bfloat16 else MOE_F32
    else:
        _dev(out, "out", FP8, (max_rows, N // 2))
        _dev(out_scales, "out_scales", torch.float32, (max_rows, N // 2 // 128))
        code = MOE_FP8_E4M3
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_grouped_gemm_fp8_noalloc(_p(a), _p(as_), _p(offsets), G, max_rows, _p(b_t), b_layout, _p(bs), N,
                                              K, epilogue, mode, tile_rows, _p(out), code, _p(out_scales),
                                              _stream(stream)), "moe_grouped_gemm_fp8_noalloc")
    return out if epilogue == MOE_EPI_STORE else (out, out_scales)


def moe_combine(y: torch.Tensor, dest_row: torch.Tensor, topk_w: torch.Tensor, shared_first_row: Optional[torch.Tensor] = None,
                out_dtype=None, out=None, stream=None) -> torch.Tensor:
    """out[t] = sum_j w[t,j] y[dest_row[t,j]] (+ y[shared_first_row + t]); shared_first_row is a
    one-element device int32 view (e.g. offsets[E:E+1])."""
    _dev(y, "y", (torch.float32, torch.bfloat16))
    T, k = dest_row.shape
    H = y.shape[1]
    _dev(dest_row, "dest_row", torch.int32)
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if shared_first_row is not None:
        _dev(shared_first_row, "shared_first_row", torch.int32, (1,))
    od = y.dtype if out_dtype is None else out_dtype
    out = torch.empty((T, H), dtype=od, device=y.device) if out is None else _dev(out, "out", od, (T, H))
    _check(lib().moe_combine(_p(y), _act_code(y), _p(dest_row), _p(topk_w), T, k, H, _p(shared_first_row), _p(out),
                             _act_code(out), _stream(stream)), "moe_combine")
    return out


def moe_combine_residual(y: torch.Tensor, dest_row: torch.Tensor, topk_w: torch.Tensor,
                         shared_first_row: Optional[torch.Tensor], residual: torch.Tensor, x_next=None, out=None,
                         write_out: bool = False, stream=None):
    """The combine on a residual branch: o = act(sum_j w[t,j] y[dest_row[t,j]] (+ shared row)) and
    x_next = act(residual + o), act = residual's dtype.  Returns x_next, or (x_next, o) when
    ``write_out`` (o then goes to ``out``, bitwise what moe_combine writes).  x_next may be
    ``residual`` itself (in-place update of the stack's activations)."""
    _dev(y, "y", (torch.float32, torch.bfloat16))
    T, k = dest_row.shape
    H = y.shape[1]
    _dev(dest_row, "dest_row", torch.int32)
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if shared_first_row is not None:
        _dev(shared_first_row, "shared_first_row", torch.int32, (1,))
    _dev(residual, "residual", (torch.float32, torch.bfloat16), (T, H))
    ad = residual.dtype
    x_next = torch.empty_like(residual) if x_next is None else _dev(x_next, "x_next", ad, (T, H))
    if write_out:
        out = torch.empty((T, H), dtype=ad, device=y.device) if out is None else _dev(out, "out", ad, (T, H))
    else:
        out = None
    _check(lib().moe_combine_residual(_p(y), _act_code(y), _p(dest_row), _p(topk_w), T, k, H, _p(shared_first_row),
                                      _p(residual), _p(out), _p(x_next), _act_code(residual), _stream(stream)),
           "moe_combine_residual")
    return (x_next, out) if write_out else x_next


def payload_bytes(n: int, num_experts: int) -> int:
    """Bytes of a packed router-replay payload of n indices (0 for an invalid size)."""
    return int(lib().moe_payload_bytes(n, num_experts))


def _payload_out(n: int, num_experts: int, out, device):
    nb = payload_bytes(n, num_experts)
    if nb == 0 and n != 0:
        raise MoeError(MOE_ERR_SHAPE, "moe_payload_bytes")
    if out is None:
        return torch.empty(nb, dtype=torch.uint8, device=device)
    if out.dtype != torch.uint8 or out.numel() < nb or not out.is_contiguous():
        raise ValueError(f"packed buffer must be contiguous uint8 with >= {nb} bytes")
    return out


def moe_payload_pack(payload: torch.Tensor, num_experts: int, out: Optional[torch.Tensor] = None,
                     bad_count: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Bit-pack a router-replay payload (any shape of int32 indices, e.g. [num_layers, top_k, seq_len])
    to ceil(log2 E) bits per index; returns the packed uint8 device buffer."""
    _dev(payload, "payload", torch.int32)
    if bad_count is not None:
        _dev(bad_count, "bad_count", torch.int32, (1,))
    n = payload.numel()
    out = _payload_out(n, num_experts, out, payload.device)
    if out.device.type != "cuda":
        raise ValueError("packed buffer must be on the GPU")
    _check(lib().moe_payload_pack(_p(payload), n, num_experts, _p(out), _p(bad_count), _stream(stream)),
           "moe_payload_pack")
    return out


def moe_payload_unpack(packed: torch.Tensor, shape, num_experts: int, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Inverse of moe_payload_pack: int32 indices of the given shape."""
    _dev(packed, "packed", torch.uint8)
    n = 1
    for d in shape:
        n *= int(d)
    if packed.numel() < payload_bytes(n, num_experts):
        raise ValueError("packed buffer smaller than moe_payload_bytes")
    out = torch.empty(tuple(shape), dtype=torch.int32, device=packed.device) if out is None else \
        _dev(out, "out", torch.int32, tuple(shape))
    _check(lib().moe_payload_unpack(_p(packed), n, num_experts, _p(out), _stream(stream)), "moe_payload_unpack")
    return out


def moe_payload_to_host(payload: torch.Tensor, num_experts: int, staging: torch.Tensor, host: torch.Tensor,
                        bad_count: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack on the device into `staging` and copy the packed bytes into `host` (a pinned uint8 CPU
    tensor) asynchronously on the stream; returns `host`."""
    _dev(payload, "payload", torch.int32)
    n = payload.numel()
    nb = payload_bytes(n, num_experts)
    _payload_out(n, num_experts, staging, payload.device)
    if host.device.type != "cpu" or host.dtype != torch.uint8 or host.numel() < nb or not host.is_contiguous():
        raise ValueError(f"host buffer must be a contiguous uint8 CPU tensor with >= {nb} bytes")
    if not host.is_pinned():
        raise ValueError("host buffer must be pinned (torch.empty(..., pin_memory=True)): the copy is asynchronous")
    _check(lib().moe_payload_to_host(_p(payload), n, num_experts, _p(staging), _p(host), _p(bad_count),
                                     _stream(stream)), "moe_payload_to_host")
    return host


def moe_payload_from_host(host: torch.Tensor, shape, num_experts: int, staging: torch.Tensor,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Copy packed bytes from `host` (pinned uint8 CPU tensor) to `staging` and unpack them on the
    device, asynchronously on the stream."""
    n = 1
    for d in shape:
        n *= int(d)
    nb = payload_bytes(n, num_experts)
    if host.device.type != "cpu" or host.dtype != torch.uint8 or host.numel() < nb or not host.is_contiguous():
        raise ValueError(f"host buffer must be a contiguous uint8 CPU tensor with >= {nb} bytes")
    if not host.is_pinned():
        raise ValueError("host buffer must be pinned (torch.empty(..., pin_memory=True)): the copy is asynchronous")
    _dev(staging, "staging", torch.uint8)
    _payload_out(n, num_experts, staging, staging.device)
    out = torch.empty(tuple(shape), dtype=torch.int32, device=staging.device) if out is None else \
        _dev(out, "out", torch.int32, tuple(shape))
    _check(lib().moe_payload_from_host(_p(host), n, num_experts, _p(staging), _p(out), _stream(stream)),
           "moe_payload_from_host")
    return out



# ----------------------------------------------------------------------------- backward
def moe_combine_backward(dout: torch.Tensor, y: torch.Tensor, dest_row: torch.Tensor, topk_w: torch.Tensor,
                         shared_first_row: Optional[torch.Tensor] = None, pow2: bool = False, dyq=None, dys=None,
                         dw=None, row_w: Optional[torch.Tensor] = None, stream=None):
    """dY = w * dout per slot row (dout for the shared row), 1x128-quantised into (dyq [rows,H] uint8,
    dys [rows,H/128] fp32) with rows = y.shape[0], and dw[t,j] = <dout[t], y[dest_row[t,j]]> (fp32 [T,k]).
    row_w: optional fp32 [rows] that receives each written row's factor."""
    _dev(dout, "dout", (torch.float32, torch.bfloat16))
    _dev(y, "y", (torch.float32, torch.bfloat16))
    T, k = dest_row.shape
    rows, H = y.shape
    _dev(dout, "dout", shape=(T, H))
    _dev(dest_row, "dest_row", torch.int32)
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if shared_first_row is not None:
        _dev(shared_first_row, "shared_first_row", torch.int32, (1,))
    dev = y.device
    dyq = torch.empty((rows, H), dtype=FP8, device=dev) if dyq is None else _dev(dyq, "dyq", FP8, (rows, H))
    dys = torch.empty((rows, H // 128), dtype=torch.float32, device=dev) if dys is None else \
        _dev(dys, "dys", torch.float32, (rows, H // 128))
    dw = torch.empty((T, k), dtype=torch.float32, device=dev) if dw is None else _dev(dw, "dw", torch.float32, (T, k))
    if row_w is not None:
        _dev(row_w, "row_w", torch.float32, (rows,))
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_combine_backward(_p(dout), _act_code(dout), _p(y), _act_code(y), _p(dest_row), _p(topk_w), T, k, H,
                                      _p(shared_first_row), mode, _p(dyq), _p(dys), _p(dw), _p(row_w),
                                      _stream(stream)), "moe_combine_backward")
    return dyq, dys, dw


def moe_swiglu_backward_quant(dh: torch.Tensor, g: torch.Tensor, pow2: bool = False, dgq=None, dgs=None, stream=None):
    """dG = [dgate | dup] of h = silu(gate) * up (g = [gate | up] [rows,2F] fp32, dh [rows,F] fp32),
    1x128-quantised: (dgq [rows,2F] uint8, dgs [rows,2F/128] fp32)."""
    rows, F = dh.shape
    _dev(dh, "dh", torch.float32)
    _dev(g, "g", torch.float32, (rows, 2 * F))
    dgq = torch.empty((rows, 2 * F), dtype=FP8, device=dh.device) if dgq is None else _dev(dgq, "dgq", FP8, (rows, 2 * F))
    dgs = torch.empty((rows, 2 * F // 128), dtype=torch.float32, device=dh.device) if dgs is None else \
        _dev(dgs, "dgs", torch.float32, (rows, 2 * F // 128))
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_swiglu_backward_quant(_p(dh), _p(g), rows, F, mode, _p(dgq), _p(dgs), _stream(stream)),
           "moe_swiglu_backward_quant")
    return dgq, dgs


def moe_route_backward(logits: torch.Tensor, topk_idx: torch.Tensor, dw: torch.Tensor, cfg: RouterCfg, dz=None,
                       stream=None) -> torch.Tensor:
    """dz [T,E] fp32: gradient of the logits from the routing-weight gradient dw, selection fixed."""
    T, E = logits.shape
    k = cfg.top_k
    _dev(logits, "logits", torch.float32)
    _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(dw, "dw", torch.float32, (T, k))
    if E != cfg.num_experts:
        raise ValueError("logits width != num_experts")
    dz = torch.empty((T, E), dtype=torch.float32, device=logits.device) if dz is None else \
        _dev(dz, "dz", torch.float32, (T, E))
    _check(lib().moe_route_backward(_p(logits), _p(topk_idx), _p(dw), T, ctypes.byref(cfg), _p(dz), _stream(stream)),
           "moe_route_backward")
    return dz


def gate_backward_workspace(T: int, E: int, H: int) -> int:
    return int(lib().moe_gate_backward_workspace(T, E, H))


def moe_gate_backward(dz: torch.Tensor, x: torch.Tensor, wg: torch.Tensor, dx_in: Optional[torch.Tensor] = None,
                      dx_dtype=None, dx=None, dwg=None, db=None, want_db: bool = True, workspace=None, stream=None):
    """dx = dx_in + dz Wg (rounded once to dx_dtype), dWg = dz^T x, db = column sums of dz (fp32).
    Returns (dx, dwg, db or None)."""
    T, H = x.shape
    E = wg.shape[0]
    _dev(dz, "dz", torch.float32, (T, E))
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(wg, "wg", torch.float32, (E, H))
    if dx_in is not None:
        _dev(dx_in, "dx_in", torch.float32, (T, H))
    dev = x.device
    od = x.dtype if dx_dtype is None else dx_dtype
    dx = torch.empty((T, H), dtype=od, device=dev) if dx is None else _dev(dx, "dx", od, (T, H))
    dwg = torch.empty((E, H), dtype=torch.float32, device=dev) if dwg is None else _dev(dwg, "dwg", torch.float32, (E, H))
    if want_db:
        db = torch.empty(E, dtype=torch.float32, device=dev) if db is None else _dev(db, "db", torch.float32, (E,))
    else:
        db = None
    need = gate_backward_workspace(T, E, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    _check(lib().moe_gate_backward(_p(dz), _p(x), _act_code(x), _p(wg), T, H, E, _p(dx_in), _p(dx), _act_code(dx),
                                   _p(dwg), _p(db), _p(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "moe_gate_backward")
    return dx, dwg, db


def wgrad_max_tiles(max_rows: int, groups: int) -> int:
    """128-row tiles the weight-gradient operands are sized for."""
    return int(lib().moe_wgrad_max_tiles(max_rows, groups))


def moe_wgrad_tiles(offsets: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tile_first [G+1] int32: each group's first 128-row tile of the weight-gradient operands."""
    G = offsets.shape[0] - 1
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    out = torch.empty(G + 1, dtype=torch.int32, device=offsets.device) if out is None else \
        _dev(out, "tile_first", torch.int32, (G + 1,))
    _check(lib().moe_wgrad_tiles(_p(offsets), G, _p(out), _stream(stream)), "moe_wgrad_tiles")
    return out


def _colwise_out(C, max_tiles, qt, st, dev):
    qt = torch.empty((C, max_tiles * 128), dtype=FP8, device=dev) if qt is None else \
        _dev(qt, "qt", FP8, (C, max_tiles * 128))
    st = torch.empty((C, max_tiles), dtype=torch.float32, device=dev) if st is None else \
        _dev(st, "st", torch.float32, (C, max_tiles))
    return qt, st


def moe_colwise_quant_rows(x: torch.Tensor, offsets: torch.Tensor, tile_first: torch.Tensor, max_tiles: int,
                           src_row: Optional[torch.Tensor] = None, row_scale: Optional[torch.Tensor] = None,
                           pow2: bool = False, qt=None, st=None, stream=None):
    """128x1-quantised transposed operand: column c, row r = row_scale[r] * x[src_row[r], c], each
    group's rows in whole 128-row tiles.  Returns (codes, scales) buffers of C * max_tiles * 128 bytes
    and C * max_tiles floats (shaped [C, max_tiles*128] / [C, max_tiles] for storage only): group g's
    codes are the row-major [C, 128 n_g] block at flat offset tile_first[g] * 128 * C, its scales the
    [C, n_g] block at tile_first[g] * C (``colwise_block``)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    C = x.shape[1]
    G = offsets.shape[0] - 1
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    _dev(tile_first, "tile_first", torch.int32, (G + 1,))
    if src_row is not None:
        _dev(src_row, "src_row", torch.int32)
    if row_scale is not None:
        _dev(row_scale, "row_scale", torch.float32)
    qt, st = _colwise_out(C, max_tiles, qt, st, x.device)
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_colwise_quant_rows(_p(x), _act_code(x), _p(src_row), _p(row_scale), _p(offsets), _p(tile_first),
                                        G, max_tiles, C, mode, _p(qt), _p(st), _stream(stream)),
           "moe_colwise_quant_rows")
    return qt, st


def colwise_block(qt: torch.Tensor, st: torch.Tensor, tile_first, g: int):
    """Views of group g's codes [C, 128 n_g] and scales [C, n_g] in a column-wise operand buffer
    (tile_first: host sequence of int)."""
    C = qt.shape[0]
    t0, t1 = int(tile_first[g]), int(tile_first[g + 1])
    q = qt.reshape(-1)[t0 * 128 * C:t1 * 128 * C].view(C, (t1 - t0) * 128)
    s = st.reshape(-1)[t0 * C:t1 * C].view(C, t1 - t0)
    return q, s


def moe_colwise_quant_swiglu(g: torch.Tensor, offsets: torch.Tensor, tile_first: torch.Tensor, max_tiles: int,
                             dh: Optional[torch.Tensor] = None, pow2: bool = False, qt=None, st=None, stream=None):
    """128x1-quantised transposed h = silu(gate) * up (dh None; C = F) or dG = [dgate | dup] (C = 2F)
    from the GEMM1 output g [rows, 2F] fp32."""
    rows, F2 = g.shape
    F = F2 // 2
    _dev(g, "g", torch.float32)
    if dh is not None:
        _dev(dh, "dh", torch.float32, (rows, F))
    G = offsets.shape[0] - 1
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    _dev(tile_first, "tile_first", torch.int32, (G + 1,))
    qt, st = _colwise_out(F2 if dh is not None else F, max_tiles, qt, st, g.device)
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_colwise_quant_swiglu(_p(g), _p(dh), F, _p(offsets), _p(tile_first), G, max_tiles, mode, _p(qt),
                                          _p(st), _stream(stream)), "moe_colwise_quant_swiglu")
    return qt, st


def moe_grouped_gemm_wgrad(a: torch.Tensor, as_: torch.Tensor, b: torch.Tensor, bs: torch.Tensor,
                           tile_first: torch.Tensor, max_tiles: int, pow2: bool = False, out=None, stream=None):
    """out[g] = A_g B_g^T over group g's tiles: a [M, max_tiles*128], b [N, max_tiles*128] codes with
    scales [M, max_tiles], [N, max_tiles] -> fp32 [G, M, N]."""
    M, N = a.shape[0], b.shape[0]
    G = tile_first.shape[0] - 1
    _dev(a, "a", FP8, (M, max_tiles * 128))
    _dev(b, "b", FP8, (N, max_tiles * 128))
    _dev(as_, "as", torch.float32, (M, max_tiles))
    _dev(bs, "bs", torch.float32, (N, max_tiles))
    _dev(tile_first, "tile_first", torch.int32, (G + 1,))
    out = torch.empty((G, M, N), dtype=torch.float32, device=a.device) if out is None else \
        _dev(out, "out", torch.float32, (G, M, N))
    mode = MOE_SCALE_POW2 if pow2 else MOE_SCALE_AMAX
    _check(lib().moe_grouped_gemm_wgrad(_p(a), _p(as_), M, _p(b), _p(bs), N, _p(tile_first), G, max_tiles, mode,
                                        _p(out), _stream(stream)), "moe_grouped_gemm_wgrad")
    return out


def moe_transpose_fp8_blocks(q: torch.Tensor, scales: torch.Tensor, qt=None, scales_t=None, stream=None):
    """[G,N,K] 128x128-block codes and [G,N/128,K/128] scales -> ([G,K,N], [G,K/128,N/128])."""
    _dev(q, "q", FP8)
    G, N, K = q.shape
    _dev(scales, "scales", torch.float32, (G, N // 128, K // 128))
    qt = torch.empty((G, K, N), dtype=FP8, device=q.device) if qt is None else _dev(qt, "qt", FP8, (G, K, N))
    scales_t = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device=q.device) if scales_t is None else \
        _dev(scales_t, "scales_t", torch.float32, (G, K // 128, N // 128))
    _check(lib().moe_transpose_fp8_blocks(_p(q), _p(scales), G, N, K, _p(qt), _p(scales_t), _stream(stream)),
           "moe_transpose_fp8_blocks")
    return qt, scales_t

from .layer import (MoELayerWeights, MoELayer, BackwardWeights, pack_expert_weights,  # noqa: E402,F401
                    prepare_backward_weights, quantize_expert_weights)
