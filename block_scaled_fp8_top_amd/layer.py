"""One MoE layer forward composed from the C-ABI calls, with buffers allocated once.

forward(x) enqueues, on the current stream and without any host synchronisation:
  moe_gate_logits -> moe_route_quant (the router, optionally recording into the routing payload, and
  the 1x128 quantisation of x in one launch) or moe_replay_route / moe_replay_gate ->
  moe_quant_fp8_block (x, 1x128) -> moe_dispatch_plan (permutation indices and
  scales, and the tile plan of both expert GEMMs) -> moe_grouped_gemm_fp8_gather (W1 on the rows of
  xq gathered through src_token, SwiGLU + 1x128 quantisation of h) -> moe_grouped_gemm_fp8_planned
  (W2) -> moe_combine.
forward_chunks(xs, outs) runs independent token chunks through the same forward, each chunk's gate
projection (after the first) on a second stream beside the previous chunk's combine.

backward(x, dout, bw) enqueues the gradients of the last forward (its buffers must still hold its
results): moe_combine_backward (dY codes, dw) -> moe_grouped_gemm_fp8 (dY, W2^T: dh) ->
moe_grouped_gemm_fp8 (A, W1: the GEMM1 output recomputed, unless a training forward kept it) ->
moe_swiglu_backward_quant (dG codes)
-> moe_grouped_gemm_fp8 (dG, W1^T: dA) -> moe_combine (dA, weights 1: expert part of dx) ->
moe_route_backward (dz) -> moe_gate_backward (dx, dWg, db).

This is the layer that "RL at 1T Scale: prime-rl Performance Deep Dive" runs in FP8 at inference
(section "FP8 inference") and in block-scaled FP8 in the trainer (section "FP8 training"), with
router replay (section "Router replay") as a mode of the same forward.  Its forward also takes FP4
expert weights (E2M1 in 1x32 blocks with E8M0 scales, the activations staying FP8 with power-of-two
1x128 scales): the 4-bit variant the page lists as future work (section "Future work").
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import torch

import block_scaled_fp8_top_amd as M


@dataclass
class MoELayerWeights:
    """Router gate and 128x128-block-quantised expert weights (group E is the shared expert).
    The forward streams the packed copies (w1p, w2p) when present, else the row-major codes.
    FP4 experts (see quantize_expert_weights_fp4) come only packed, as PackedWeightFP4 in w1p and
    w2p with their own scales, and need pow2 (the activations' scales are then powers of two)."""
    wg: torch.Tensor                 # [E,H] fp32
    bias: Optional[torch.Tensor]     # [E] fp32
    w1q: Optional[torch.Tensor]      # [G,2F,H] e4m3 bytes (None once packed without a row-major copy)
    w1s: Optional[torch.Tensor]      # [G,2F/128,H/128] fp32 (None for FP4 experts)
    w2q: Optional[torch.Tensor]      # [G,H,F] e4m3 bytes
    w2s: Optional[torch.Tensor]      # [G,H/128,F/128] fp32 (None for FP4 experts)
    cfg: M.RouterCfg
    shared: bool
    w1p: Optional[M.PackedWeight | M.PackedWeightFP4] = None   # w1 packed for the SwiGLU epilogue
    w2p: Optional[M.PackedWeight | M.PackedWeightFP4] = None   # w2 packed for the store epilogue
    pow2: bool = False                     # power-of-two block scales: the weights were quantised so,
                                           # and the forward quantises x and h the same way

    @property
    def E(self) -> int:
        return int(self.cfg.num_experts)

    @property
    def H(self) -> int:
        return int(self.wg.shape[1])

    @property
    def fp4(self) -> bool:
        return isinstance(self.w1p, M.PackedWeightFP4)

    @property
    def F(self) -> int:
        return int(self.w2p.K) if self.fp4 else int(self.w2s.shape[2]) * 128

    @property
    def groups(self) -> int:
        return int(self.w1p.G) if self.fp4 else int(self.w1s.shape[0])


def pack_expert_weights(weights: MoELayerWeights, keep_rowmajor: bool = True, stream=None) -> MoELayerWeights:
    """Weights with packed copies of w1 (SwiGLU panels) and w2 (store panels) for the grouped GEMM;
    without ``keep_rowmajor`` the row-major codes are dropped."""
    w1p = M.moe_pack_weights_fp8(weights.w1q, M.MOE_EPI_SWIGLU_QUANT, stream=stream)
    w2p = M.moe_pack_weights_fp8(weights.w2q, M.MOE_EPI_STORE, stream=stream)
    if keep_rowmajor:
        return replace(weights, w1p=w1p, w2p=w2p)
    return replace(weights, w1q=None, w2q=None, w1p=w1p, w2p=w2p)


@dataclass
class BackwardWeights:
    """The expert-weight copies the backward streams, all packed for the store epilogue: W1 as is
    (the GEMM1 output is recomputed rather than kept), and W1^T, W2^T (128x128 blocks transposed
    together with their scales, so no re-quantisation)."""
    w1_store: M.PackedWeight   # W1 [G,2F,H]
    w1t: M.PackedWeight        # W1^T [G,H,2F]
    w1ts: torch.Tensor         # [G,H/128,2F/128]
    w2t: M.PackedWeight        # W2^T [G,F,H]
    w2ts: torch.Tensor         # [G,F/128,H/128]


def prepare_backward_weights(weights: MoELayerWeights, stream=None) -> BackwardWeights:
    """Transposed and store-packed copies of the expert weights (from the row-major codes)."""
    if weights.w1q is None or weights.w2q is None:
        raise ValueError("prepare_backward_weights needs the row-major codes (pack with keep_rowmajor=True)")
    w1t, w1ts = M.moe_transpose_fp8_blocks(weights.w1q, weights.w1s, stream=stream)
    w1t_p = M.moe_pack_weights_fp8(w1t, M.MOE_EPI_STORE, stream=stream)
    del w1t
    w2t, w2ts = M.moe_transpose_fp8_blocks(weights.w2q, weights.w2s, stream=stream)
    w2t_p = M.moe_pack_weights_fp8(w2t, M.MOE_EPI_STORE, stream=stream)
    del w2t
    w1_store = M.moe_pack_weights_fp8(weights.w1q, M.MOE_EPI_STORE, stream=stream)
    return BackwardWeights(w1_store, w1t_p, w1ts, w2t_p, w2ts)


def quantize_expert_weights(groups: int, H: int, F: int, master, device="cuda", stream=None, pow2: bool = False):
    """Allocate the quantised weight tensors and fill expert g from ``master(g) -> (w1 [2F,H], w2 [H,F])``
    (fp32 or bf16 device tensors), one expert at a time so the fp32 masters never coexist; pow2:
    power-of-two block scales."""
    w1q = torch.empty((groups, 2 * F, H), dtype=torch.uint8, device=device)
    w1s = torch.empty((groups, 2 * F // 128, H // 128), dtype=torch.float32, device=device)
    w2q = torch.empty((groups, H, F), dtype=torch.uint8, device=device)
    w2s = torch.empty((groups, H // 128, F // 128), dtype=torch.float32, device=device)
    for g in range(groups):
        w1, w2 = master(g)
        M.moe_quant_fp8_block(w1, 128, q=w1q[g], scales=w1s[g], stream=stream, pow2=pow2)
        M.moe_quant_fp8_block(w2, 128, q=w2q[g], scales=w2s[g], stream=stream, pow2=pow2)
    return w1q, w1s, w2q, w2s


def quantize_expert_weights_fp4(groups: int, H: int, F: int, master, device="cuda", stream=None):
    """FP4 expert weights, the 4-bit variant: expert g from ``master(g) -> (w1 [2F,H], w2 [H,F])``
    (fp32 or bf16 device tensors) is quantised to FP4 E2M1 in 1x32 blocks along the input
    dimension with E8M0 scales (moe_quant_mxfp4), one expert at a time, and the codes are packed
    for the two GEMM epilogues.  Returns (w1p, w2p) as PackedWeightFP4, for MoELayerWeights with
    w1q = w1s = w2q = w2s = None and pow2=True."""
    w1q = torch.empty((groups, 2 * F, H // 2), dtype=torch.uint8, device=device)
    w1e = torch.empty((groups, 2 * F, H // 32), dtype=torch.uint8, device=device)
    w2q = torch.empty((groups, H, F // 2), dtype=torch.uint8, device=device)
    w2e = torch.empty((groups, H, F // 32), dtype=torch.uint8, device=device)
    for g in range(groups):
        w1, w2 = master(g)
        M.moe_quant_mxfp4(w1, q=w1q[g], e8=w1e[g], stream=stream)
        M.moe_quant_mxfp4(w2, q=w2q[g], e8=w2e[g], stream=stream)
    w1p = M.moe_pack_weights_fp4(w1q, w1e, M.MOE_EPI_SWIGLU_QUANT, stream=stream)
    w2p = M.moe_pack_weights_fp4(w2q, w2e, M.MOE_EPI_STORE, stream=stream)
    return w1p, w2p


class MoELayer:
    """Preallocated buffers for up to ``T_max`` tokens; ``forward`` returns a view of the output."""

    def __init__(self, weights: MoELayerWeights, T_max: int, act_dtype=torch.bfloat16, device="cuda",
                 gather_rows: bool = True, tile_rows: int = 0):
        """gather_rows: GEMM1 reads each group row's codes straight from the token-order xq through
        the dispatch's src_token (only the scales are permuted); False: the dispatch also writes the
        permuted codes (disp.aq) and GEMM1 reads those.  Both give bitwise the same results.
        tile_rows: row-tile height of the expert GEMMs (0: chosen from the group sizes)."""
        if weights.fp4 and not weights.pow2:
            raise ValueError("FP4 expert weights need power-of-two activation scales (pow2=True)")
        self.w = weights
        self.T_max = T_max
        self.act = act_dtype
        E, H, F, k = weights.E, weights.H, weights.F, int(weights.cfg.top_k)
        G = weights.groups
        self.max_rows = T_max * k + (T_max if weights.shared else 0)
        d = device
        self.logits = torch.empty((T_max, E), dtype=torch.float32, device=d)
        self.idx = torch.empty((T_max, k), dtype=torch.int32, device=d)
        self.wts = torch.empty((T_max, k), dtype=torch.float32, device=d)
        self.xq = torch.empty((T_max, H), dtype=torch.uint8, device=d)
        self.xs = torch.empty((T_max, H // 128), dtype=torch.float32, device=d)
        self.disp = M.Dispatched(
            counts=torch.empty(G, dtype=torch.int32, device=d),
            offsets=torch.empty(G + 1, dtype=torch.int32, device=d),
            dest_row=torch.empty((T_max, k), dtype=torch.int32, device=d),
            src_token=torch.empty(self.max_rows, dtype=torch.int32, device=d),
            aq=None if gather_rows else torch.empty((self.max_rows, H), dtype=torch.uint8, device=d),
            as_=torch.empty((self.max_rows, H // 128), dtype=torch.float32, device=d),
            max_rows=self.max_rows)
        self.hq = torch.empty((self.max_rows, F), dtype=torch.uint8, device=d)
        self.hs = torch.empty((self.max_rows, F // 128), dtype=torch.float32, device=d)
        self.y = torch.empty((self.max_rows, H), dtype=act_dtype, device=d)
        self.out = torch.empty((T_max, H), dtype=act_dtype, device=d)
        self.workspace = torch.empty(M.workspace_bytes(M.MOE_OP_DISPATCH, T_max, k, E), dtype=torch.uint8, device=d)
        self.gemm_ws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, self.max_rows, 0, G, 0, 0),
                                   dtype=torch.uint8, device=d)
        self.bad = torch.zeros(1, dtype=torch.int32, device=d)
        self.plan = None   # tile plan of the last forward's expert GEMMs
        self.logits_valid = False   # the last forward wrote self.logits (not the fused sigmoid replay)
        self.device = d
        self.gather_rows = gather_rows
        self.tile_rows = tile_rows
        self.bwd = None    # backward buffers, allocated by the first backward (or training forward)
        self.g_saved = False   # the last forward kept GEMM1's output in self.bwd["g"]
        self._side = None      # second stream of forward_chunks (default priority), made on first use

    def _gemm1_a(self):
        """GEMM1's A operand: (codes, group-order scales)."""
        return (self.xq if self.gather_rows else self.disp.aq), self.disp.as_

    def _a_rows(self):
        return self.disp.src_token if self.gather_rows else None

    def forward(self, x: torch.Tensor, replay: Optional[torch.Tensor] = None, record: Optional[torch.Tensor] = None,
                stream=None, events=None, fused_replay: bool = True, training: bool = False,
                out: Optional[torch.Tensor] = None, residual_out: Optional[torch.Tensor] = None,
                _gate_done: bool = False, _before_combine=None) -> torch.Tensor:
        """``events``: optional list of 7 timing events (torch.cuda.Event), recorded on the launch
        stream before the first stage and after each of the six stages (gate logits, routing with
        x's quantisation, dispatch, GEMM1, GEMM2, combine).  With ``replay`` and a
        sigmoid router the gate projection and the replay run fused (``fused_replay``), and
        ``self.logits`` is not written.  ``training``: GEMM1 also keeps its fp32 output for the
        backward (which then does not recompute it).  ``out``: where the combine writes the layer
        output (default: the layer's own buffer), e.g. a chunk's rows of a longer sequence.
        ``residual_out``: the layer sits on a residual branch; the combine then writes
        act(x + output) there (it may be x itself) and returns it, and the layer output itself is
        written only if ``out`` is given.  (``_gate_done`` and ``_before_combine`` serve
        forward_chunks: the logits of x are already in place; a call made once the second GEMM is
        enqueued.)"""
        T = x.shape[0]
        if T != self.T_max:
            raise ValueError(f"layer buffers are sized for T={self.T_max}, got {T}")
        w = self.w
        if training and w.fp4:
            raise ValueError("FP4 expert weights are an inference format here: no training forward or backward")
        st = torch.cuda.current_stream() if stream is None else stream

        def mark(i):
            if events is not None:
                events[i].record(st)

        mark(0)
        fused = replay is not None and int(w.cfg.score_fn) == M.MOE_SCORE_SIGMOID and fused_replay
        self.logits_valid = not fused
        if not fused and not _gate_done:
            M.moe_gate_logits(x, w.wg, w.bias, out=self.logits, stream=stream)
        mark(1)
        # routing stage: the routing decisions and x's 1x128 quantisation
        if fused:
            # sigmoid replay: only the k recorded logits per token are needed (logits is not written)
            M.moe_replay_gate(x, w.wg, w.bias, w.cfg, replay, bad_count=self.bad, topk_idx=self.idx, topk_w=self.wts,
                              stream=stream)
        elif replay is not None:
            M.moe_replay_route(self.logits, w.cfg, replay, bad_count=self.bad, topk_idx=self.idx, topk_w=self.wts,
                               stream=stream)
        else:
            # the router and x's 1x128 quantisation in one launch
            M.moe_route_quant(self.logits, w.cfg, x, record=record, topk_idx=self.idx, topk_w=self.wts, q=self.xq,
                              scales=self.xs, stream=stream, pow2=w.pow2)
        if replay is not None:
            M.moe_quant_fp8_block(x, 1, q=self.xq, scales=self.xs, stream=stream, pow2=w.pow2)
        mark(2)
        # dispatch, and one tile plan for both expert GEMMs (same groups), living in the GEMM workspace
        # (for decode-sized batches the dispatch workgroup writes it)
        plan = self.plan = M.moe_dispatch_plan(self.idx, w.E, w.shared, self.xq, self.xs, self.workspace, self.disp,
                                               self.gemm_ws, tile_rows=self.tile_rows, stream=stream)
        mark(3)
        M.moe_grouped_gemm_fp8(*self._gemm1_a(), self.disp.offsets, w.w1p or w.w1q, w.w1s,
                               epilogue=M.MOE_EPI_SWIGLU_QUANT, out=self.hq, out_scales=self.hs, plan=plan,
                               stream=stream, pow2=w.pow2,
                               save_g=self._backward_buffers()["g"] if training else None, a_rows=self._a_rows())
        self.g_saved = training
        mark(4)
        M.moe_grouped_gemm_fp8(self.hq, self.hs, self.disp.offsets, w.w2p or w.w2q, w.w2s, epilogue=M.MOE_EPI_STORE,
                               out_dtype=self.act, out=self.y, plan=plan, stream=stream, pow2=w.pow2)
        mark(5)
        if _before_combine is not None:
            _before_combine()
        shared_row = self.disp.offsets[w.E:w.E + 1] if w.shared else None
        if residual_out is not None:
            res = M.moe_combine_residual(self.y, self.disp.dest_row, self.wts, shared_row, x, x_next=residual_out,
                                         out=out, write_out=out is not None, stream=stream)
            mark(6)
            return res[0] if out is not None else res
        o = self.out if out is None else out
        M.moe_combine(self.y, self.disp.dest_row, self.wts, shared_row, out=o, stream=stream)
        mark(6)
        return o

    def forward_chunks(self, xs, outs, stream=None):
        """Forward of independent token chunks in order (each of T_max tokens, e.g. the chunks of a
        long sequence's prefill), chunk c's output into outs[c]; returns outs.  Chunk c + 1's gate
        projection runs on a second stream while chunk c's combine runs: the projection is fp32
        VALU work and the combine a stream through HBM, so they overlap, and the logits buffer the
        projection writes has been read by chunk c's router once chunk c's second GEMM is done.
        Chunk c + 1's router waits for both.  Every chunk's results are forward(xs[c])'s, bit for
        bit.  Inference only: no replay, recording, training forward or residual form."""
        main = torch.cuda.current_stream() if stream is None else stream
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
        side, n = self._side, len(xs)
        if len(outs) != n:
            raise ValueError("one output per chunk")
        gemm2_done = [torch.cuda.Event() for _ in range(n)]
        gate_done = [torch.cuda.Event() for _ in range(n)]
        for c in range(n):
            hook = None
            if c + 1 < n:
                def hook(c=c):
                    gemm2_done[c].record(main)
                    side.wait_event(gemm2_done[c])
                    M.moe_gate_logits(xs[c + 1], self.w.wg, self.w.bias, out=self.logits, stream=side)
                    gate_done[c + 1].record(side)
            if c > 0:
                main.wait_event(gate_done[c])
            self.forward(xs[c], stream=main, out=outs[c], _gate_done=c > 0, _before_combine=hook)
        return outs

    def _backward_buffers(self):
        if self.bwd is not None:
            return self.bwd
        w, d, R, T = self.w, self.device, self.max_rows, self.T_max
        E, H, F, k = w.E, w.H, w.F, int(w.cfg.top_k)
        f32 = torch.float32
        self.bwd = dict(
            dyq=torch.empty((R, H), dtype=torch.uint8, device=d), dys=torch.empty((R, H // 128), dtype=f32, device=d),
            dw=torch.empty((T, k), dtype=f32, device=d), dh=torch.empty((R, F), dtype=f32, device=d),
            g=torch.empty((R, 2 * F), dtype=f32, device=d), dgq=torch.empty((R, 2 * F), dtype=torch.uint8, device=d),
            dgs=torch.empty((R, 2 * F // 128), dtype=f32, device=d), dA=torch.empty((R, H), dtype=f32, device=d),
            ones=torch.ones((T, k), dtype=f32, device=d), dx_exp=torch.empty((T, H), dtype=f32, device=d),
            dz=torch.empty((T, E), dtype=f32, device=d), dx=torch.empty((T, H), dtype=self.act, device=d),
            dwg=torch.empty((E, H), dtype=f32, device=d), db=torch.empty(E, dtype=f32, device=d),
            gws=torch.empty(max(M.gate_backward_workspace(T, E, H), 1), dtype=torch.uint8, device=d),
            row_w=torch.empty(R, dtype=f32, device=d))
        return self.bwd

    def _wgrad_buffers(self):
        b = self._backward_buffers()
        if "dW1" in b:
            return b
        w, d = self.w, self.device
        H, F, G = w.H, w.F, w.groups
        mt = M.wgrad_max_tiles(self.max_rows, G)
        kp, f32, u8 = mt * 128, torch.float32, torch.uint8
        b.update(max_tiles=mt, tile_first=torch.empty(G + 1, dtype=torch.int32, device=d),
                 dYt=torch.empty((H, kp), dtype=u8, device=d), dYts=torch.empty((H, mt), dtype=f32, device=d),
                 ht=torch.empty((F, kp), dtype=u8, device=d), hts=torch.empty((F, mt), dtype=f32, device=d),
                 dGt=torch.empty((2 * F, kp), dtype=u8, device=d), dGts=torch.empty((2 * F, mt), dtype=f32, device=d),
                 xt=torch.empty((H, kp), dtype=u8, device=d), xts=torch.empty((H, mt), dtype=f32, device=d),
                 dW1=torch.empty((G, 2 * F, H), dtype=f32, device=d), dW2=torch.empty((G, H, F), dtype=f32, device=d))
        return b

    def backward(self, x: torch.Tensor, dout: torch.Tensor, bw: BackwardWeights, stream=None, events=None,
                 weight_grads: bool = False) -> dict:
        """Gradients of the last forward (x is that forward's input) for the output gradient dout [T,H]
        (activation dtype): dx [T,H] (activation dtype), dwg [E,H] and db [E] (None without a bias)
        in fp32, plus the routing-weight gradient dw [T,k] and the logit gradient dz [T,E]; with
        ``weight_grads`` also the expert-weight gradients dW1 [G,2F,H] and dW2 [G,H,F] (fp32).  The
        returned tensors are views of buffers reused by the next backward.  ``events``: optional
        list of 9 timing events (11 with weight_grads) recorded before the first and after each stage."""
        if self.plan is None:
            raise RuntimeError("backward needs a forward first")
        if self.w.fp4:
            raise ValueError("FP4 expert weights are an inference format here: no backward")
        if x.shape[0] != self.T_max or tuple(dout.shape) != (self.T_max, self.w.H):
            raise ValueError("x / dout do not match the layer's buffers")
        w = self.w
        b = self._wgrad_buffers() if weight_grads else self._backward_buffers()
        st = torch.cuda.current_stream() if stream is None else stream

        def mark(i):
            if events is not None:
                events[i].record(st)

        off = self.disp.offsets
        shared_row = off[w.E:w.E + 1] if w.shared else None
        mark(0)
        M.moe_combine_backward(dout, self.y, self.disp.dest_row, self.wts, shared_row, pow2=w.pow2, dyq=b["dyq"],
                               dys=b["dys"], dw=b["dw"], row_w=b["row_w"] if weight_grads else None, stream=stream)
        mark(1)
        M.moe_grouped_gemm_fp8(b["dyq"], b["dys"], off, bw.w2t, bw.w2ts, epilogue=M.MOE_EPI_STORE,
                               out_dtype=torch.float32, out=b["dh"], plan=self.plan, stream=stream, pow2=w.pow2)
        mark(2)
        if not self.g_saved:
            M.moe_grouped_gemm_fp8(*self._gemm1_a(), off, bw.w1_store, w.w1s, epilogue=M.MOE_EPI_STORE,
                                   out_dtype=torch.float32, out=b["g"], plan=self.plan, stream=stream, pow2=w.pow2,
                                   a_rows=self._a_rows())
        mark(3)
        M.moe_swiglu_backward_quant(b["dh"], b["g"], pow2=w.pow2, dgq=b["dgq"], dgs=b["dgs"], stream=stream)
        mark(4)
        M.moe_grouped_gemm_fp8(b["dgq"], b["dgs"], off, bw.w1t, bw.w1ts, epilogue=M.MOE_EPI_STORE,
                               out_dtype=torch.float32, out=b["dA"], plan=self.plan, stream=stream, pow2=w.pow2)
        mark(5)
        M.moe_combine(b["dA"], self.disp.dest_row, b["ones"], shared_row, out_dtype=torch.float32, out=b["dx_exp"],
                      stream=stream)
        mark(6)
        if not self.logits_valid:
            M.moe_gate_logits(x, w.wg, w.bias, out=self.logits, stream=stream)
            self.logits_valid = True
        M.moe_route_backward(self.logits, self.idx, b["dw"], w.cfg, dz=b["dz"], stream=stream)
        mark(7)
        M.moe_gate_backward(b["dz"], x, w.wg, dx_in=b["dx_exp"], dx_dtype=self.act, dx=b["dx"], dwg=b["dwg"],
                            db=b["db"], want_db=w.bias is not None, workspace=b["gws"], stream=stream)
        mark(8)
        res = dict(dx=b["dx"], dwg=b["dwg"], db=b["db"] if w.bias is not None else None, dw=b["dw"], dz=b["dz"])
        if weight_grads:
            # 128x1 operands over each expert's rows, then one fp32 matrix per expert
            mt, tf, src = b["max_tiles"], b["tile_first"], self.disp.src_token
            M.moe_wgrad_tiles(off, out=tf, stream=stream)
            M.moe_colwise_quant_rows(dout, off, tf, mt, src_row=src, row_scale=b["row_w"], pow2=w.pow2, qt=b["dYt"],
                                     st=b["dYts"], stream=stream)
            M.moe_colwise_quant_swiglu(b["g"], off, tf, mt, pow2=w.pow2, qt=b["ht"], st=b["hts"], stream=stream)
            M.moe_colwise_quant_swiglu(b["g"], off, tf, mt, dh=b["dh"], pow2=w.pow2, qt=b["dGt"], st=b["dGts"],
                                       stream=stream)
            M.moe_colwise_quant_rows(x, off, tf, mt, src_row=src, pow2=w.pow2, qt=b["xt"], st=b["xts"], stream=stream)
            mark(9)
            M.moe_grouped_gemm_wgrad(b["dYt"], b["dYts"], b["ht"], b["hts"], tf, mt, pow2=w.pow2, out=b["dW2"],
                                     stream=stream)
            M.moe_grouped_gemm_wgrad(b["dGt"], b["dGts"], b["xt"], b["xts"], tf, mt, pow2=w.pow2, out=b["dW1"],
                                     stream=stream)
            mark(10)
            res.update(dW1=b["dW1"], dW2=b["dW2"])
        return res
