"""CPU oracle of the MoE layer backward (gradients of the block-scaled FP8 layer).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): imported by ``tests/`` and ``bench.py``'s
CPU baseline leg, never by the product package, and it shares no code with the HIP library.

"RL at 1T Scale: prime-rl Performance Deep Dive", section "FP8 training": the trainer runs the
same block-scaled FP8 recipe as inference (DeepSeek V3's), so the layer's backward contracts in
FP8 too; section "Router replay": the trainer replays the recorded routing, so the expert
selection is a fixed input of the backward and only the routing weights carry gradient.  The
pages give no formula for any of it; the readings used here:

* Combine backward.  With out[t] = sum_j w[t,j] Y[dest(t,j)] + Y_shared[t]: the row gradient is
  dY[dest(t,j)] = w[t,j] * dout[t] (one fp32 product of the stored values), dY of a shared row is
  dout[t]; the routing-weight gradient is dw[t,j] = <dout[t], Y[dest(t,j)]> over Y as stored
  (activation dtype).  Slots routed nowhere (index -1) get dw = 0 and no row.
* Activation gradients are quantised like the forward's activations: 1x128 blocks along the
  contraction dimension of the next GEMM (H for dY, 2F for dG), with the layer's scale rule.
* Data-gradient GEMMs use the forward's 128x128 weight blocks transposed together with their
  scales (exact: a block's scale is shared by all its elements): dh = deq(dY) deq(W2),
  dA = deq(dG) deq(W1), fp32 accumulation on the device, fp64 here.
* SwiGLU backward from the GEMM1 output G = [gate | up] (recomputed, not stored):
  s = sigmoid(gate), dgate = dh * up * s * (1 + gate (1 - s)), dup = dh * gate * s; rounded to
  fp32, then quantised.
* dx = sum_j dA[dest(t,j)] + dA_shared[t] + dz[t] Wg: the expert part in slot order, the shared
  row last, then the router part.
* Expert-weight gradients: dW2[e] = sum over e's rows r of dY[r]^T h[r] ([H,F]) and
  dW1[e] = sum over e's rows of dG[r]^T x[r] ([2F,H]), with h = silu(gate) up in fp32 from the
  GEMM1 output and x the layer input row (activation dtype) of the row's token.  Both operands of
  these products contract over rows, so they are quantised in 128x1 blocks: 128 consecutive rows of
  one expert by one column (the expert's rows zero-padded to a multiple of 128), i.e. 1x128 blocks
  of the transposed segment; fp32 accumulation, fp32 result.
* Router backward (selection fixed): sigmoid scores s = 1 / (1 + exp(-z)); softmax scores are
  the full softmax over E.  Renormalised weights w_j = score_j / sum_l score_l:
      sigmoid:  dz_{i_j} = s_j (1 - s_j) (dw_j - sum_l w_l dw_l) / sum_l s_l
      softmax:  dz_{i_j} = w_j (dw_j - sum_l w_l dw_l)        (the full-softmax denominator cancels)
  Not renormalised (w_j = score_j):
      sigmoid:  dz_{i_j} = dw_j s_j (1 - s_j)
      softmax:  dz_e = [e selected] w_e dw_e - p_e sum_l w_l dw_l   (dense over all E)
  dz is the gradient of the logit including the bias, so db = sum_t dz[t] and dWg = dz^T x.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

import oracle as O


def combine_backward(dout: np.ndarray, y_act: np.ndarray, dest: np.ndarray, w: np.ndarray,
                     rows: int, shared_row0: Optional[int] = None):
    """Row gradients dY [rows,H] (fp32: the fp32 product w * dout) and dw [T,k] (fp64)."""
    dout32 = np.asarray(dout, np.float32)
    T, k = dest.shape
    H = dout32.shape[1]
    dY = np.zeros((rows, H), np.float32)
    dw = np.zeros((T, k), np.float64)
    y64 = np.asarray(y_act, np.float64)
    for j in range(k):
        d = dest[:, j]
        ok = d >= 0
        dY[d[ok]] = np.asarray(w, np.float32)[ok, j][:, None] * dout32[ok]
        dw[ok, j] = np.einsum("th,th->t", dout32[ok].astype(np.float64), y64[d[ok]])
    if shared_row0 is not None:
        dY[shared_row0:shared_row0 + T] = dout32
    return dY, dw


def swiglu_backward(dh: np.ndarray, g1: np.ndarray, F: int) -> np.ndarray:
    """dG = [dgate | dup] for h = silu(gate) * up, gate = g1[:, :F], up = g1[:, F:2F]; fp64 -> fp32."""
    dh = np.asarray(dh, np.float64)
    g = np.asarray(g1, np.float64)
    gate, up = g[:, :F], g[:, F:2 * F]
    s = 1.0 / (1.0 + np.exp(-gate))
    dgate = dh * up * s * (1.0 + gate * (1.0 - s))
    dup = dh * gate * s
    return np.concatenate([dgate, dup], axis=1).astype(np.float32)


def route_backward(z: np.ndarray, idx: np.ndarray, dw: np.ndarray, cfg: O.RouterCfg) -> np.ndarray:
    """dz [T,E] (fp64) from the routing-weight gradient dw [T,k], selection idx held fixed."""
    z = np.asarray(z, np.float64)
    T, E = z.shape
    dz = np.zeros((T, E), np.float64)
    for t in range(T):
        sel = [j for j in range(idx.shape[1]) if idx[t, j] >= 0]
        if not sel:
            continue
        e = np.array([int(idx[t, j]) for j in sel])
        g = np.array([float(dw[t, j]) for j in sel])
        if cfg.score_fn == O.SIGMOID:
            s = 1.0 / (1.0 + np.exp(-z[t, e]))
            if cfg.renormalize:
                S = s.sum()
                wt = s / S
                dz[t, e] = s * (1.0 - s) * (g - np.dot(wt, g)) / S
            else:
                dz[t, e] = g * s * (1.0 - s)
        else:
            p = np.exp(z[t] - z[t].max())
            p /= p.sum()
            if cfg.renormalize:
                wt = p[e] / p[e].sum()
                dz[t, e] = wt * (g - np.dot(wt, g))
            else:
                wt = p[e]
                dz[t] = -p * np.dot(wt, g)
                dz[t, e] += wt * g
    return dz


def colwise_segments(a32: np.ndarray, offsets, quant: bool = True, pow2: bool = False):
    """Per group g: rows offsets[g]..offsets[g+1] of a [rows, C], zero-padded to a multiple of 128
    rows and transposed to [C, Kg]; with quant, 1x128-quantised along Kg (= 128x1 blocks of a).
    Returns a list of (codes, scales) or, without quant, of fp64 [C, Kg] values."""
    out = []
    a32 = np.asarray(a32, np.float32)
    C = a32.shape[1]
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        kg = -(-(r1 - r0) // 128) * 128
        seg = np.zeros((kg, C), np.float32)
        seg[:r1 - r0] = a32[r0:r1]
        segT = np.ascontiguousarray(seg.T)
        out.append(O.moe_quant_fp8_block(segT, 1, pow2) if quant else segT.astype(np.float64))
    return out


def wgrad(dY: np.ndarray, h: np.ndarray, dG: np.ndarray, xrows: np.ndarray, offsets, quant: bool = True,
          pow2: bool = False):
    """dW2[g] = dY_g^T h_g ([H,F]) and dW1[g] = dG_g^T x_g ([2F,H]) over each group's rows, in fp64
    from the 128x1-quantised operands (or the fp32 values without quant)."""
    def val(seg):
        return O.dequant_act(*seg) if quant else seg
    sY, sh = colwise_segments(dY, offsets, quant, pow2), colwise_segments(h, offsets, quant, pow2)
    sG, sx = colwise_segments(dG, offsets, quant, pow2), colwise_segments(xrows, offsets, quant, pow2)
    dW2 = np.stack([val(a) @ val(b).T for a, b in zip(sY, sh)])
    dW1 = np.stack([val(a) @ val(b).T for a, b in zip(sG, sx)])
    return dW1, dW2


def gate_backward(dz: np.ndarray, x: np.ndarray, wg: np.ndarray):
    """dx_router = dz Wg [T,H], dWg = dz^T x [E,H], db = column sums of dz [E] (fp64)."""
    dz = np.asarray(dz, np.float64)
    return dz @ np.asarray(wg, np.float64), dz.T @ np.asarray(x, np.float64), dz.sum(axis=0)


def _deq_or_keep(a32: np.ndarray, quant: bool, pow2: bool):
    """1x128 quantisation of an fp32 activation gradient and its fp64 value (or the fp32 value)."""
    if not quant:
        return None, None, np.asarray(a32, np.float64)
    q, s = O.moe_quant_fp8_block(a32, 1, pow2)
    return q, s, O.dequant_act(q, s)


def backward_core(dout, x, z, idx, w, dest, offsets, y_act, g1, cfg: O.RouterCfg, wg,
                  w1: Sequence[np.ndarray], w2: Sequence[np.ndarray], F: int, shared: bool,
                  act: str = "f32", quant: bool = True, pow2: bool = False, src=None) -> dict:
    """The whole backward over all tokens, in the dispatch (expert-grouped) layout.

    w1[g], w2[g]: fp64 values of group g's weights ([2F,H], [H,F]: dequantised codes, or the
    masters when quant is off); g1: the forward's GEMM1 output [rows,2F]; y_act: the forward's
    stored expert rows.  With quant off every quantisation is skipped (the plain real-valued
    chain rule of the same layer), which is what the autograd pin compares against."""
    T, k = dest.shape
    E = cfg.num_experts
    rows = int(offsets[-1])
    dY, dw = combine_backward(dout, y_act, dest, w, rows, int(offsets[E]) if shared else None)
    dYq, dYs, dYd = _deq_or_keep(dY, quant, pow2)
    H = dY.shape[1]
    G = len(w1)
    dh = np.zeros((rows, F), np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            dh[r0:r1] = dYd[r0:r1] @ w2[g]
    dG = swiglu_backward(dh, g1, F)
    dGq, dGs, dGd = _deq_or_keep(dG, quant, pow2)
    dA = np.zeros((rows, H), np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            dA[r0:r1] = dGd[r0:r1] @ w1[g]
    dx_exp = O.moe_combine(dA, dest, np.ones((T, k), np.float32),
                           dA[int(offsets[E]):int(offsets[E]) + T] if shared else None)
    dz = route_backward(z, idx, dw, cfg)
    dx_r, dwg, db = gate_backward(dz, x, wg)
    res = dict(dY=dY, dYq=dYq, dYs=dYs, dw=dw, dh=dh, dG=dG, dGq=dGq, dGs=dGs, dA=dA,
               dx_experts=dx_exp, dz=dz, dx_router=dx_r, dx=dx_exp + dx_r, dwg=dwg, db=db)
    if src is not None:
        h = np.asarray(g1, np.float64)
        h = (h[:, :F] / (1.0 + np.exp(-h[:, :F])) * h[:, F:2 * F]).astype(np.float32)
        xrows = np.asarray(x, np.float32)[np.asarray(src)[:rows]]
        res["dW1"], res["dW2"] = wgrad(dY, h, dG, xrows, offsets, quant, pow2)
    return res


def backward_dispatch(layer, fwd: dict, x: np.ndarray, dout: np.ndarray) -> dict:
    """Backward of ``oracle.layer.forward_dispatch``'s result ``fwd`` for the output gradient dout."""
    G = layer.groups
    w1 = [O.dequant_weight(layer.get(g).w1q, layer.get(g).w1s) for g in range(G)]
    w2 = [O.dequant_weight(layer.get(g).w2q, layer.get(g).w2s) for g in range(G)]
    return backward_core(dout, x, fwd["z"], fwd["idx"], fwd["w"], fwd["dest"], fwd["offsets"], fwd["y_act"],
                         fwd["g1"], layer.cfg, layer.wg, w1, w2, layer.F, layer.shared, layer.act,
                         quant=True, pow2=layer.pow2, src=fwd["src"])


def backward_token(layer, x_rows: np.ndarray, dout_rows: np.ndarray, replay_rows=None) -> dict:
    """Per-token backward of sampled tokens with no dispatch: each token's rows are formed,
    quantised and pushed through its own experts directly (a token's expert-path gradient
    depends on that token alone).  Returns dw, dz, dx_experts, dx_router, dx for the rows."""
    import oracle.layer as OL
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x_rows, layer.wg, layer.bias)
    idx, w, _ = OL.route_or_replay(layer, z, replay_rows)
    xq, xs = O.moe_quant_fp8_block(x_rows, 1, layer.pow2)
    n, H = x_rows.shape
    k = idx.shape[1]
    dout32 = np.asarray(dout_rows, np.float32)
    dw = np.zeros((n, k), np.float64)
    dx_exp = np.zeros((n, H), np.float64)
    for t in range(n):
        slots = [(j, int(idx[t, j]), np.float32(w[t, j])) for j in range(k) if idx[t, j] >= 0]
        if layer.shared:
            slots.append((None, E, np.float32(1.0)))
        for j, e, we in slots:
            ew = layer.get(e)
            g1, _, _, _, _, y_act = OL.expert_ffn(ew, xq[t:t + 1], xs[t:t + 1], F, layer.act, layer.pow2)
            if j is not None:
                dw[t, j] = float(np.dot(dout32[t].astype(np.float64), y_act[0].astype(np.float64)))
            dY = (we * dout32[t:t + 1]).astype(np.float32)
            dYq, dYs = O.moe_quant_fp8_block(dY, 1, layer.pow2)
            dh = O.dequant_act(dYq, dYs) @ O.dequant_weight(ew.w2q, ew.w2s)
            dG = swiglu_backward(dh, g1, F)
            dGq, dGs = O.moe_quant_fp8_block(dG, 1, layer.pow2)
            dx_exp[t] += (O.dequant_act(dGq, dGs) @ O.dequant_weight(ew.w1q, ew.w1s))[0]
    dz = route_backward(z, idx, dw, layer.cfg)
    dx_r = dz @ np.asarray(layer.wg, np.float64)
    return dict(z=z, idx=idx, w=w, dw=dw, dz=dz, dx_experts=dx_exp, dx_router=dx_r, dx=dx_exp + dx_r)


def wgrad_expert(layer, x: np.ndarray, dout: np.ndarray, e: int, replay=None):
    """dW1 and dW2 of expert e alone over a whole batch (x, dout [T,H]): the batch is routed, e's rows
    are formed in dispatch order (ascending token) and evaluated row by row (each row depends on its
    own token only), then contracted as in ``wgrad``.  Returns (dW1 [2F,H], dW2 [H,F]) fp64."""
    import oracle.layer as OL
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x, layer.wg, layer.bias)
    idx, w, _ = OL.route_or_replay(layer, z, replay)
    dout32 = np.asarray(dout, np.float32)
    if e == E:
        toks = np.arange(x.shape[0])
        fac = np.ones(len(toks), np.float32)
    else:
        t_, j_ = np.nonzero(idx == e)
        order = np.argsort(t_, kind="stable")
        toks, fac = t_[order], np.asarray(w, np.float32)[t_[order], j_[order]]
    ew = layer.get(e)
    xr = np.asarray(x, np.float32)[toks]
    xq, xs = O.moe_quant_fp8_block(xr, 1, layer.pow2)
    g1 = O.dequant_act(xq, xs) @ O.dequant_weight(ew.w1q, ew.w1s).T
    h = O.swiglu(g1, F)
    dY = (fac[:, None] * dout32[toks]).astype(np.float32)
    dYq, dYs = O.moe_quant_fp8_block(dY, 1, layer.pow2)
    dh = O.dequant_act(dYq, dYs) @ O.dequant_weight(ew.w2q, ew.w2s)
    dG = swiglu_backward(dh, g1, F)
    dW1, dW2 = wgrad(dY, h, dG, xr, [0, len(toks)], True, layer.pow2)
    return dW1[0], dW2[0]
