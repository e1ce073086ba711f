"""CPU oracle for the block-scaled FP8 Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py``; never by the product package.  It shares no code with the HIP
library.

The method is the MoE layer of "RL at 1T Scale: prime-rl Performance Deep Dive" (Prime
Intellect blog): top-k routing, or router replay of routing indices recorded at inference in a
``[num_layers, top_k, seq_len]`` payload (section "Router replay"); dispatch of tokens into
per-expert groups and the weighted combine back (sections "Wide EP", "Parallelism / EP");
block-scaled FP8 quantisation as proposed by DeepSeek V3 feeding FP8 expert GEMMs (sections
"FP8 inference", "FP8 training").  The pages print no formula for these steps; the readings
used here are fixed in the C file ``moe_oracle.c`` (bit-exact fp32 parts) and below (fp64
parts), one function per step.

Bit-exact steps (logits, router, replay, quantisation, dispatch) run in the C file; the
tolerance-checked steps (GEMMs, SwiGLU, combine) run here in fp64 with numpy, whose matrix
product is the library primitive used for the contraction.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None
_lock = threading.Lock()

SOFTMAX, SIGMOID = 0, 1


def build(force: bool = False) -> str:
    """Compile the C part with gcc (fp32 ops in program order: no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64, I32 = ctypes.c_int64, ctypes.c_int32
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
        lib.orc_exp.restype = ctypes.c_float
        lib.orc_exp.argtypes = [ctypes.c_float]
        lib.orc_sigmoid.restype = ctypes.c_float
        lib.orc_sigmoid.argtypes = [ctypes.c_float]
        lib.orc_exp_array.argtypes = [P, I64, P]
        lib.orc_sigmoid_array.argtypes = [P, I64, P]
        lib.orc_gate_logits.argtypes = [P, P, P, I64, I32, I32, P]
        lib.orc_route.argtypes = [P, I64, P, P, P, P, I64]
        lib.orc_replay_route.restype = I64
        lib.orc_replay_route.argtypes = [P, I64, P, P, I64, P, P]
        lib.orc_quant_block.argtypes = [P, I64, I64, I32, I32, I32, P, P]
        lib.orc_pow2_scale.restype = ctypes.c_float
        lib.orc_pow2_scale.argtypes = [ctypes.c_float]
        lib.orc_dispatch.argtypes = [P, I64, I32, I32, I32, P, P, P, P]
        lib.orc_permute_rows.argtypes = [P, P, I64, I64, P]
        lib.orc_dequant_act.argtypes = [P, P, I64, I32, P]
        lib.orc_dequant_weight.argtypes = [P, P, I32, I32, P]
        lib.orc_gemm_block_form.argtypes = [P, P, I64, P, P, I32, I32, P]
        lib.orc_e2m1_value.restype = ctypes.c_double
        lib.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_encode.restype = ctypes.c_uint8
        lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
        lib.orc_e2m1_encode_array.argtypes = [P, I64, P]
        lib.orc_fp4_scale.restype = ctypes.c_float
        lib.orc_fp4_scale.argtypes = [ctypes.c_float]
        lib.orc_quant_mxfp4.argtypes = [P, I64, I32, P, P]
        lib.orc_dequant_mxfp4.argtypes = [P, P, I64, I32, P]
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class RouterCfg(ctypes.Structure):
    """Router configuration; field meanings as in the C file."""
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("group_score_topk", ctypes.c_int32)]


def router_cfg(num_experts, top_k, score_fn, renormalize, n_group=1, topk_group=1, group_score_topk=2):
    if n_group > 1:
        assert num_experts % n_group == 0 and n_group <= 1024 and num_experts // n_group <= 1024
        assert 1 <= topk_group <= n_group and 1 <= group_score_topk <= num_experts // n_group
        assert top_k <= topk_group * (num_experts // n_group)
    assert 1 <= top_k <= num_experts
    return RouterCfg(num_experts, top_k, score_fn, int(bool(renormalize)), n_group, topk_group, group_score_topk)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ------------------------------------------------------------------ bf16 helpers (exact)
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 (given as uint16 bit patterns) to fp32; exact."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def round_to_bf16(x) -> np.ndarray:
    """fp64/fp32 -> fp32 -> bf16, returned widened to fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


# ------------------------------------------------------------------ FP8 e4m3
def e4m3_value(code: int) -> float:
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_table() -> np.ndarray:
    """fp64 value of every code 0..255 (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


# ------------------------------------------------------------------ pinned exp / sigmoid
def pinned_exp(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _load().orc_exp_array(_ptr(x), x.size, _ptr(out))
    return out


def pinned_sigmoid(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _load().orc_sigmoid_array(_ptr(x), x.size, _ptr(out))
    return out


# ------------------------------------------------------------------ the seven steps
def moe_gate_logits(x_f32: np.ndarray, wg: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """z[t,e] = fp32 fma chain over h ascending (+ bias).  x: [T,H] fp32 (bf16 widened)."""
    x = _c(x_f32, np.float32)
    wg = _c(wg, np.float32)
    T, H = x.shape
    E = wg.shape[0]
    assert wg.shape == (E, H)
    b = None if bias is None else _c(bias, np.float32)
    z = np.empty((T, E), np.float32)
    _load().orc_gate_logits(_ptr(x), _ptr(wg), None if b is None else _ptr(b), T, H, E, _ptr(z))
    return z


def moe_route(z: np.ndarray, cfg: RouterCfg, record: np.ndarray | None = None):
    """Top-k routing.  Returns (idx [T,k] int32, w [T,k] fp32).  If ``record`` ([k, >=T] int32,
    one layer of the payload) is given it is filled in place with record[j, t] = idx[t, j]."""
    z = _c(z, np.float32)
    T = z.shape[0]
    assert z.shape[1] == cfg.num_experts
    k = cfg.top_k
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rec_ptr, rec_ld = None, 0
    if record is not None:
        assert record.dtype == np.int32 and record.flags.c_contiguous and record.shape[0] == k and record.shape[1] >= T
        rec_ptr, rec_ld = _ptr(record), record.shape[1]
    _load().orc_route(_ptr(z), T, ctypes.byref(cfg), _ptr(idx), _ptr(w), rec_ptr, rec_ld)
    return idx, w


def moe_replay_route(z: np.ndarray, cfg: RouterCfg, replay: np.ndarray):
    """Replay recorded indices (replay: [k, >=T] int32).  Returns (idx, w, bad_count)."""
    z = _c(z, np.float32)
    replay = _c(replay, np.int32)
    T = z.shape[0]
    k = cfg.top_k
    assert replay.shape[0] == k and replay.shape[1] >= T
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    bad = _load().orc_replay_route(_ptr(z), T, ctypes.byref(cfg), _ptr(replay), replay.shape[1], _ptr(idx), _ptr(w))
    return idx, w, int(bad)


def pow2_scale(amax: float) -> float:
    """Power-of-two block scale of a block whose largest magnitude is amax (see the C file)."""
    return float(_load().orc_pow2_scale(float(amax)))


def moe_quant_fp8_block(x_f32: np.ndarray, block_rows: int, pow2: bool = False):
    """Block quantisation of x ([rows, cols] or [batch, rows, cols], fp32); with pow2 the scales are
    powers of two (the smallest at or above amax / 448).
    Returns (codes uint8 same shape, scales fp32 [..., rows/block_rows, cols/128])."""
    x = _c(x_f32, np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    B, R, C = x.shape
    assert C % 128 == 0 and R % block_rows == 0 and block_rows in (1, 128)
    q = np.empty(x.shape, np.uint8)
    s = np.empty((B, R // block_rows, C // 128), np.float32)
    _load().orc_quant_block(_ptr(x), B, R, C, block_rows, 1 if pow2 else 0, _ptr(q), _ptr(s))
    if squeeze:
        return q[0], s[0]
    return q, s


def moe_dispatch(idx: np.ndarray, num_experts: int, append_shared: bool):
    """Stable counting sort of expert ids.  Returns counts [G], offsets [G+1], dest_row [T,k],
    src_token [rows] (G = E + shared)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    G = num_experts + (1 if append_shared else 0)
    counts = np.zeros(G, np.int32)
    offsets = np.zeros(G + 1, np.int32)
    dest = np.empty((T, k), np.int32)
    n_valid = int((idx >= 0).sum())
    rows = n_valid + (T if append_shared else 0)
    src = np.empty(rows, np.int32)
    _load().orc_dispatch(_ptr(idx), T, k, num_experts, int(bool(append_shared)), _ptr(counts), _ptr(offsets),
                         _ptr(dest), _ptr(src))
    return counts, offsets, dest, src


def permute_rows(x: np.ndarray, src_token: np.ndarray) -> np.ndarray:
    """out[row] = x[src_token[row]] (x: [T, ...] any dtype)."""
    x = np.ascontiguousarray(x)
    src = _c(src_token, np.int32)
    out = np.empty((src.shape[0],) + x.shape[1:], x.dtype)
    row_bytes = x[0].nbytes if x.shape[0] else 0
    _load().orc_permute_rows(_ptr(x.view(np.uint8)), _ptr(src), src.shape[0], row_bytes, _ptr(out.view(np.uint8)))
    return out


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 value of 1x128-scaled codes q [M,K] with scales [M,K/128] (exact)."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    M, K = q.shape
    assert s.shape == (M, K // 128)
    out = np.empty((M, K), np.float64)
    _load().orc_dequant_act(_ptr(q), _ptr(s), M, K, _ptr(out))
    return out


def dequant_weight(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 value of 128x128-scaled codes q [N,K] with scales [N/128,K/128] (exact)."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    N, K = q.shape
    assert s.shape == (N // 128, K // 128)
    out = np.empty((N, K), np.float64)
    _load().orc_dequant_weight(_ptr(q), _ptr(s), N, K, _ptr(out))
    return out


def gemm_block_form(aq, as_, bq, bs) -> np.ndarray:
    """Block-scaled product in its defining per-128-K-block form (fp64)."""
    aq, as_ = _c(aq, np.uint8), _c(as_, np.float32)
    bq, bs = _c(bq, np.uint8), _c(bs, np.float32)
    M, K = aq.shape
    N = bq.shape[0]
    out = np.empty((M, N), np.float64)
    _load().orc_gemm_block_form(_ptr(aq), _ptr(as_), M, _ptr(bq), _ptr(bs), N, K, _ptr(out))
    return out


def moe_grouped_gemm_fp8(aq, as_, offsets, bq, bs) -> np.ndarray:
    """Grouped block-scaled GEMM in fp64: for each group g, rows offsets[g]..offsets[g+1] of
    deq(a) times deq(b[g])^T.  aq [rows,K], as_ [rows,K/128], bq [G,N,K], bs [G,N/128,K/128]."""
    offsets = np.asarray(offsets)
    G, N, K = bq.shape
    rows = aq.shape[0]
    out = np.zeros((rows, N), np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            out[r0:r1] = dequant_act(aq[r0:r1], as_[r0:r1]) @ dequant_weight(bq[g], bs[g]).T
    return out


def swiglu(g: np.ndarray, F: int) -> np.ndarray:
    """h = silu(gate) * up with gate = g[:, :F], up = g[:, F:2F]; fp64, rounded to fp32."""
    g = np.asarray(g, np.float64)
    gate, up = g[:, :F], g[:, F:2 * F]
    return (gate / (1.0 + np.exp(-gate)) * up).astype(np.float32)


def moe_combine(y: np.ndarray, dest_row: np.ndarray, w: np.ndarray, y_shared: np.ndarray | None = None):
    """out[t] = sum_j w[t,j] * y[dest_row[t,j]] (+ y_shared[t]) in fp64; dest -1 contributes nothing."""
    y = np.asarray(y, np.float64)
    T, k = dest_row.shape
    out = np.zeros((T, y.shape[1]), np.float64)
    for j in range(k):
        d = dest_row[:, j]
        ok = d >= 0
        out[ok] += w[ok, j].astype(np.float64)[:, None] * y[d[ok]]
    if y_shared is not None:
        out += np.asarray(y_shared, np.float64)
    return out


# ------------------------------------------------------------------ FP4 weights (see the C file)
def e2m1_table() -> np.ndarray:
    """fp64 value of each of the 16 FP4 E2M1 codes."""
    return np.array([_load().orc_e2m1_value(c) for c in range(16)])


def e2m1_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def fp4_scale(amax: float) -> float:
    return float(_load().orc_fp4_scale(float(amax)))


def quant_mxfp4(x_f32: np.ndarray):
    """[..., rows, cols] fp32 -> (packed codes [..., rows, cols/2] uint8, E8M0 scale codes
    [..., rows, cols/32] uint8); 1x32 blocks along cols."""
    x = _c(x_f32, np.float32)
    cols = x.shape[-1]
    assert cols % 32 == 0
    rows = x.size // cols
    q = np.empty(x.shape[:-1] + (cols // 2,), np.uint8)
    e8 = np.empty(x.shape[:-1] + (cols // 32,), np.uint8)
    _load().orc_quant_mxfp4(_ptr(x), rows, cols, _ptr(q), _ptr(e8))
    return q, e8


def dequant_mxfp4(q: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """fp64 value of packed FP4 weights [N, K/2] with E8M0 scales [N, K/32]."""
    q, e8 = _c(q, np.uint8), _c(e8, np.uint8)
    N, K = q.shape[0], q.shape[1] * 2
    assert e8.shape == (N, K // 32)
    out = np.empty((N, K), np.float64)
    _load().orc_dequant_mxfp4(_ptr(q), _ptr(e8), N, K, _ptr(out))
    return out


def moe_grouped_gemm_fp4w(aq, as_, offsets, wq, we8) -> np.ndarray:
    """Grouped GEMM with FP4 weights in fp64: rows of group g times deq_fp4(w[g])^T.
    aq [rows,K] e4m3 codes with 1x128 scales; wq [G,N,K/2]; we8 [G,N,K/32]."""
    offsets = np.asarray(offsets)
    G, N = wq.shape[0], wq.shape[1]
    out = np.zeros((aq.shape[0], N), np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            out[r0:r1] = dequant_act(aq[r0:r1], as_[r0:r1]) @ dequant_mxfp4(wq[g], we8[g]).T
    return out
