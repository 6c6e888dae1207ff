"""Forward and backward pass of one MoE layer, composed from the C-ABI calls.

Every arithmetic step runs in the HIP library; this module only owns the
device buffers (allocated once through torch) and sequences the calls on one
stream (two with ``overlap_wgrad``).  No host synchronisation happens inside a pass: the per-expert
offsets produced by counting stay on the device and are read there by the
grouped GEMMs.

Forward (expert selection, then expert computation [Summary, Method details /
technical framework]; counting, indexing and the grouped GEMM [Brief, Core
method]):

    logits = x @ wr                    moe_grouped_gemm_fwd (one group, fp32 out)
    idx, w, p = top-k softmax          moe_route_topk
    counts, offsets, dest, src         moe_count_index
    xp[dest] = x (xp = x[src // k])    moe_permute
    h  = xp @ W1[e]                    moe_grouped_gemm_swiglu_fwd (one launch;
    a  = silu(h_gate) * h_up             with fuse_act=False: moe_grouped_gemm_fwd
                                         then moe_act_fwd)
    yp = a @ W2[e]                     moe_grouped_gemm_fwd
    y  = sum_j w * yp[dest]            moe_unpermute

Backward of <y, dy> (the forward-plus-backward unit of [Brief, Key results]):

    dyp, dw   moe_unpermute_bwd           da        moe_grouped_gemm_bwd
    dh        moe_act_bwd                 dW2       moe_grouped_gemm_bwd
    dxp       moe_grouped_gemm_bwd        dx_e      moe_unpermute (w = NULL)
    dW1       moe_grouped_gemm_bwd        dlogits   moe_route_topk_bwd
    dx = dx_e + dlogits @ wr^T, dwr = x^T @ dlogits   moe_grouped_gemm_bwd

With ``gather_dy`` (the default where the bf16 MFMA path applies) the
combine's gradient dyp = w * dy[src // k] is never written: the combine's
backward computes dw only, and GEMM 2's backward reads dy through the row map
with the gate weight as a row scale (moe_gather_scale,
moe_grouped_gemm_bwd_scaled_gather; its weight gradient takes the scale on
the activation, written by moe_act_bwd_scaled).
"""
from __future__ import annotations

import contextlib
import dataclasses

import torch

from . import _lib as L


@dataclasses.dataclass
class Grads:
    dx: torch.Tensor
    dwr: torch.Tensor
    dw1: torch.Tensor
    dw2: torch.Tensor


class MoELayer:
    """Buffers and call sequence for a fixed shape (T, d, E, k, F, dtype).

    ``dtype`` is ``torch.bfloat16`` (fp32 accumulation inside the kernels) or
    ``torch.float32``.  ``overlap_wgrad`` runs the two expert weight-gradient
    GEMMs on a second stream, beside the data-gradient chain; the results are
    the same bits either way.  Inputs are passed to :meth:`forward`; the returned
    tensors are views of buffers owned by the layer and are overwritten by the
    next call.

    ``recompute`` selects what the backward pass recomputes instead of reading
    it from the forward pass (selective activation checkpointing of the MoE
    layer [Brief, Core method: SAC over norm, attention and the sparse MoE]):
    ``"none"`` keeps every intermediate; ``"act"`` does not keep the SwiGLU
    output ``a`` (the backward recomputes it from ``h`` before GEMM 2's weight
    gradient); ``"layer"`` keeps only the layer's inputs (the backward re-runs
    the whole forward first).  Results are the same bits in every mode;
    :meth:`saved_bytes` gives what each mode keeps between the passes.
    """

    RECOMPUTE = ("none", "act", "layer")

    def __init__(self, T, d, E, k, F, dtype=torch.bfloat16, device="cuda", renorm=False,
                 fuse_act=True, overlap_wgrad=False, gather_x=True, recompute="none",
                 gather_dy=True):
        if not (1 <= k <= E):
            raise ValueError("need 1 <= k <= E")
        if recompute not in self.RECOMPUTE:
            raise ValueError(f"recompute must be one of {self.RECOMPUTE}")
        self.recompute = recompute
        self.T, self.d, self.E, self.k, self.F = T, d, E, k, F
        self.dtype = dtype
        self.code = L.dtype_code(dtype)
        self.renorm = bool(renorm)
        self.fuse_act = bool(fuse_act)
        self.overlap_wgrad = bool(overlap_wgrad)
        # GEMM 1 and its weight gradient read x through the row map src / k
        # instead of a permuted copy (bf16, fused activation, MFMA shapes).
        plan = L.moe_grouped_gemm_plan(3, T * k, d, 2 * F, E, self.code)
        self.gather_x = bool(gather_x) and self.fuse_act and bool(plan["mfma"])
        # GEMM 2's backward reads dy through src / k, scaled by the gate
        # weight, instead of a written dyp (bf16 MFMA shapes).
        plan2 = L.moe_grouped_gemm_plan(1, T * k, F, d, E, self.code)
        self.gather_dy = bool(gather_dy) and bool(plan2["mfma"])
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        Tk = T * k
        self.Tk = Tk
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        # routing
        self.logits = torch.empty(T, E, dtype=f32, device=dev)
        self.idx = torch.empty(T, k, dtype=i32, device=dev)
        self.w = torch.empty(T, k, dtype=f32, device=dev)
        self.probs = torch.empty(T, E, dtype=f32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.dest = torch.empty(Tk, dtype=i32, device=dev)
        self.src = torch.empty(Tk, dtype=i32, device=dev)
        self.router_offsets = torch.tensor([0, T], dtype=i32, device=dev)
        ci_ws = L.moe_count_index_workspace_size(T, k, E)
        self.ci_ws = torch.empty(max(ci_ws, 16), dtype=torch.uint8, device=dev)
        # expert activations (expert-sorted rows); the permuted copy of x
        # exists only when GEMM 1 does not gather x through src / k
        self.xp = None if self.gather_x else torch.empty(Tk, d, dtype=dtype, device=dev)
        self.h = torch.empty(Tk, 2 * F, dtype=dtype, device=dev)
        self.a = torch.empty(Tk, F, dtype=dtype, device=dev)
        self.yp = torch.empty(Tk, d, dtype=dtype, device=dev)
        self.y = torch.empty(T, d, dtype=dtype, device=dev)
        # backward
        if self.gather_dy:
            self.dyp = None
            self.w_sorted = torch.empty(Tk, dtype=f32, device=dev)
            # The backward never reads `a` here, so the scaled activation
            # takes its buffer (after backward(), `a` holds w * silu(g) * u).
            self.a_scaled = self.a
        else:
            self.dyp = torch.empty(Tk, d, dtype=dtype, device=dev)
        self.dw = torch.empty(T, k, dtype=f32, device=dev)
        self.da = torch.empty(Tk, F, dtype=dtype, device=dev)
        self.dh = torch.empty(Tk, 2 * F, dtype=dtype, device=dev)
        self.dxp = torch.empty(Tk, d, dtype=dtype, device=dev)
        self.dx_e = torch.empty(T, d, dtype=dtype, device=dev)
        self.dx = torch.empty(T, d, dtype=dtype, device=dev)
        self.dlogits = torch.empty(T, E, dtype=dtype, device=dev)
        self.dwr = torch.empty(d, E, dtype=f32, device=dev)
        self.dw1 = torch.empty(E, d, 2 * F, dtype=f32, device=dev)
        self.dw2 = torch.empty(E, F, d, dtype=f32, device=dev)
        # grouped-GEMM workspaces (split reduction partials of the weight grads)
        c = self.code
        sizes = [L.moe_grouped_gemm_workspace_size(T, d, E, 1, c),
                 L.moe_grouped_gemm_workspace_size(Tk, F, d, E, c),
                 L.moe_grouped_gemm_workspace_size(Tk, d, 2 * F, E, c)]
        self.gemm_ws_bytes = max(sizes)
        self.gemm_ws = (torch.empty(self.gemm_ws_bytes, dtype=torch.uint8, device=dev)
                        if self.gemm_ws_bytes else None)
        # Expert weight gradients on a second stream (own workspace), joined
        # at the end of backward.
        if self.overlap_wgrad:
            self.side = torch.cuda.Stream(device=dev)
            self.gemm_ws2 = (torch.empty(self.gemm_ws_bytes, dtype=torch.uint8, device=dev)
                             if self.gemm_ws_bytes else None)
            self.ev_dyp = torch.cuda.Event()
            self.ev_dh = torch.cuda.Event()
            self.ev_side = torch.cuda.Event()
        self._inputs = None
        # Optional callable name -> context manager, wrapped around every
        # library call (used by the benchmark to bracket calls with events).
        self.timer = None

    def _span(self, name):
        return self.timer(name) if self.timer is not None else contextlib.nullcontext()

    def _expect(self, t, name, shape, dtype):
        """The kernels size their buffer ranges from (T, d, E, k, F), not from
        the tensors: a tensor of another shape, dtype or device would be read
        past its end, so it is refused here."""
        if t is None:
            return
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != self.device:
            raise ValueError(f"{name}: expected {tuple(shape)} {dtype} on {self.device}, got "
                             f"{tuple(t.shape)} {t.dtype} on {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")

    # ------------------------------------------------------------------
    def forward(self, x, wr, w1, w2, bias=None, forced_idx=None, stream=None):
        T, d, E, k, F, Tk, c = self.T, self.d, self.E, self.k, self.F, self.Tk, self.code
        for t, name, shape in ((x, "x", (T, d)), (wr, "wr", (d, E)), (w1, "w1", (E, d, 2 * F)),
                               (w2, "w2", (E, F, d))):
            if t is None:
                raise ValueError(f"{name} is required")
            self._expect(t, name, shape, self.dtype)
        self._expect(bias, "bias", (E,), torch.float32)
        self._expect(forced_idx, "forced_idx", (T, k), torch.int32)
        s = stream
        with self._span("router_fwd"):
            L.moe_grouped_gemm_fwd(x, wr, self.router_offsets, T, d, E, 1, c, self.logits,
                                   L.MOE_F32, stream=s)
        with self._span("route_topk"):
            L.moe_route_topk(self.logits, bias, T, E, k, self.renorm, forced_idx, self.idx,
                             self.w, self.probs, stream=s)
        with self._span("count_index"):
            L.moe_count_index(self.idx, T, k, E, self.counts, self.offsets, self.dest, self.src,
                              self.ci_ws, self.ci_ws.numel(), stream=s)
        if not self.gather_x:
            with self._span("permute"):
                L.moe_permute(x, self.dest, T, k, d, c, self.xp, stream=s)
        if self.gather_x:
            with self._span("gemm1_swiglu_fwd"):
                L.moe_grouped_gemm_swiglu_fwd_gather(x, self.src, k, T, w1, self.offsets, Tk, d,
                                                     F, E, c, self.h, self.a, stream=s)
        elif self.fuse_act:
            with self._span("gemm1_swiglu_fwd"):
                L.moe_grouped_gemm_swiglu_fwd(self.xp, w1, self.offsets, Tk, d, F, E, c, self.h,
                                              self.a, stream=s)
        else:
            with self._span("gemm1_fwd"):
                L.moe_grouped_gemm_fwd(self.xp, w1, self.offsets, Tk, d, 2 * F, E, c, self.h, c,
                                       stream=s)
            with self._span("act_fwd"):
                L.moe_act_fwd(self.h, Tk, F, c, self.a, stream=s)
        with self._span("gemm2_fwd"):
            L.moe_grouped_gemm_fwd(self.a, w2, self.offsets, Tk, F, d, E, c, self.yp, c,
                                   stream=s)
        with self._span("unpermute"):
            L.moe_unpermute(self.yp, self.dest, self.w, T, k, d, c, self.y, stream=s)
        self._inputs = (x, wr, w1, w2, bias, forced_idx)
        return self.y

    def saved_bytes(self, recompute=None):
        """Bytes of the forward-pass results the backward pass reads (what an
        activation-memory budget must hold between the two passes), by
        tensor, for ``recompute`` (default: the layer's own mode).  The
        layer's inputs (x, weights, bias, forced ids) are not counted: the
        caller keeps them in every mode."""
        mode = self.recompute if recompute is None else recompute
        if mode not in self.RECOMPUTE:
            raise ValueError(f"recompute must be one of {self.RECOMPUTE}")
        if mode == "layer":
            return {}
        kept = {n: getattr(self, n) for n in ("probs", "idx", "w", "offsets", "dest", "src",
                                               "h", "a", "yp")}
        if mode == "act" or self.gather_dy:
            # the backward reads `a` only for GEMM 2's weight gradient, and not
            # at all when that gradient takes the scaled activation written by
            # the SwiGLU backward
            del kept["a"]
        return {n: t.numel() * t.element_size() for n, t in kept.items()}

    def capture(self, x, wr, w1, w2, dy, bias=None, forced_idx=None):
        """Record one forward + backward over these input buffers as a HIP
        graph and return it (a ``torch.cuda.CUDAGraph``): ``replay()`` re-runs
        the whole step with no per-kernel launch cost on the host.

        The graph holds the buffers' addresses, so inputs are updated in
        place between replays; results land in the layer's buffers as after
        :meth:`forward` and :meth:`backward`.  The library only enqueues
        kernels (no allocation, no memset, no host synchronisation) and this
        layer's buffers exist already, so every call of the step is
        captured.  Single-stream order only (``overlap_wgrad=False``).
        """
        if self.overlap_wgrad:
            raise ValueError("capture() records the single-stream order (overlap_wgrad=False)")
        if self.timer is not None:
            raise ValueError("capture() with a timer attached")
        main = torch.cuda.current_stream(self.device)
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(main)
        with torch.cuda.stream(side):  # one eager step off the capture
            self.forward(x, wr, w1, w2, bias=bias, forced_idx=forced_idx)
            self.backward(dy)
        main.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, wr, w1, w2, bias=bias, forced_idx=forced_idx)
            self.backward(dy)
        return graph

    def _dw1(self, x, w1, ws, wsb, stream):
        """dW1 = xp^T @ dh, with xp read from x through src / k when gathering."""
        T, d, E, k, F, Tk, c = self.T, self.d, self.E, self.k, self.F, self.Tk, self.code
        if self.gather_x:
            L.moe_grouped_gemm_bwd_gather(x, self.src, k, T, w1, self.dh, self.offsets, Tk, d,
                                          2 * F, E, c, None, None, self.dw1, ws, wsb,
                                          stream=stream)
        else:
            L.moe_grouped_gemm_bwd(self.xp, w1, self.dh, self.offsets, Tk, d, 2 * F, E, c, None,
                                   None, self.dw1, ws, wsb, stream=stream)

    def _gemm2_bwd(self, w2, ws, wsb, main, overlap):
        """GEMM 2's backward from the written dyp; the SwiGLU backward."""
        T, d, E, k, F, Tk, c = self.T, self.d, self.E, self.k, self.F, self.Tk, self.code
        if self.recompute == "act":
            # a was not kept: recompute it from the stored h (the same
            # arithmetic as GEMM 1's activation epilogue, so the same bits)
            # for GEMM 2's weight gradient.
            with self._span("act_fwd_recompute"):
                L.moe_act_fwd(self.h, Tk, F, c, self.a, stream=main)
        if overlap:
            self.ev_dyp.record(main)
        with self._span("gemm2_bwd_da"):
            # data gradient only: the activation operand `a` is not read
            L.moe_grouped_gemm_bwd(None, w2, self.dyp, self.offsets, Tk, F, d, E, c, self.da,
                                   None, None, ws, wsb, stream=main)
        with self._span("act_bwd"):
            L.moe_act_bwd(self.h, self.da, Tk, F, c, self.dh, stream=main)
        if overlap:
            self.ev_dh.record(main)
            side, ws2 = self.side, self.gemm_ws2
            side.wait_event(self.ev_dyp)
            with torch.cuda.stream(side):
                with self._span("gemm2_bwd_dw"):
                    L.moe_grouped_gemm_bwd(self.a, w2, self.dyp, self.offsets, Tk, F, d, E, c,
                                           None, None, self.dw2, ws2, wsb, stream=side)
        else:
            with self._span("gemm2_bwd_dw"):
                L.moe_grouped_gemm_bwd(self.a, w2, self.dyp, self.offsets, Tk, F, d, E, c, None,
                                       None, self.dw2, ws, wsb, stream=main)

    def _gemm2_bwd_gathered(self, dy, w2, ws, wsb, main, overlap):
        """GEMM 2's backward reading dy through src / k with the gate weight
        as a row scale (dyp is never written); the SwiGLU backward, which
        also writes the scaled activation for the weight gradient (so `a`
        itself is not read in the backward pass, whatever ``recompute``)."""
        T, d, E, k, F, Tk, c = self.T, self.d, self.E, self.k, self.F, self.Tk, self.code
        with self._span("gather_scale"):
            L.moe_gather_scale(self.w, self.src, Tk, self.w_sorted, stream=main)
        with self._span("gemm2_bwd_da"):
            L.moe_grouped_gemm_bwd_scaled_gather(None, w2, dy, self.src, k, T, self.w_sorted,
                                                 self.offsets, Tk, F, d, E, c, self.da, None,
                                                 stream=main)
        with self._span("act_bwd"):
            L.moe_act_bwd_scaled(self.h, self.da, self.w_sorted, Tk, F, c, self.dh,
                                 self.a_scaled, stream=main)
        if overlap:
            self.ev_dh.record(main)
            side, ws2 = self.side, self.gemm_ws2
            side.wait_event(self.ev_dh)
            with torch.cuda.stream(side):
                with self._span("gemm2_bwd_dw"):
                    L.moe_grouped_gemm_bwd_scaled_gather(
                        self.a_scaled, None, dy, self.src, k, T, self.w_sorted, self.offsets, Tk,
                        F, d, E, c, None, self.dw2, ws2, wsb, stream=side)
        else:
            with self._span("gemm2_bwd_dw"):
                L.moe_grouped_gemm_bwd_scaled_gather(
                    self.a_scaled, None, dy, self.src, k, T, self.w_sorted, self.offsets, Tk, F,
                    d, E, c, None, self.dw2, ws, wsb, stream=main)

    def backward(self, dy, stream=None):
        if self._inputs is None:
            raise RuntimeError("backward() before forward()")
        x, wr, w1, w2, bias, forced_idx = self._inputs
        T, d, E, k, F, Tk, c = self.T, self.d, self.E, self.k, self.F, self.Tk, self.code
        if dy is None:
            raise ValueError("dy is required")
        self._expect(dy, "dy", (T, d), self.dtype)
        s = stream
        if self.recompute == "layer":
            # Only the inputs were kept: recompute every forward result first
            # (logits, routing, indices, h, a, yp; y is rewritten unchanged).
            self.forward(x, wr, w1, w2, bias=bias, forced_idx=forced_idx, stream=s)
        ws, wsb = self.gemm_ws, self.gemm_ws_bytes
        overlap = self.overlap_wgrad and (s is None or isinstance(s, torch.cuda.Stream))
        main = (s if s is not None else torch.cuda.current_stream(self.device)) if overlap else s
        with self._span("unpermute_bwd"):
            L.moe_unpermute_bwd(dy, self.yp, self.dest, self.w, T, k, d, c, self.dyp, self.dw,
                                stream=main)
        if self.gather_dy:
            self._gemm2_bwd_gathered(dy, w2, ws, wsb, main, overlap)
        else:
            self._gemm2_bwd(w2, ws, wsb, main, overlap)
        if overlap:
            # dW1 follows dW2 on the side stream once dh exists; both fill the
            # compute units the data-gradient chain leaves idle (kernel tails,
            # memory-bound kernels).
            side = self.side
            with torch.cuda.stream(side):
                side.wait_event(self.ev_dh)
                with self._span("gemm1_bwd_dw"):
                    self._dw1(x, w1, self.gemm_ws2, wsb, side)
            self.ev_side.record(side)
        with self._span("gemm1_bwd_da"):
            # data gradient only: the activation operand `a` is not read
            L.moe_grouped_gemm_bwd(None, w1, self.dh, self.offsets, Tk, d, 2 * F, E, c,
                                   self.dxp, None, None, ws, wsb, stream=main)
        with self._span("permute_bwd"):
            L.moe_unpermute(self.dxp, self.dest, None, T, k, d, c, self.dx_e, stream=main)
        if not overlap:
            with self._span("gemm1_bwd_dw"):
                self._dw1(x, w1, ws, wsb, main)
        with self._span("route_topk_bwd"):
            L.moe_route_topk_bwd(self.probs, self.idx, self.dw, T, E, k, self.renorm,
                                 self.dlogits, c, stream=main)
        with self._span("router_bwd_da"):
            L.moe_grouped_gemm_bwd(x, wr, self.dlogits, self.router_offsets, T, d, E, 1, c,
                                   self.dx, self.dx_e, None, ws, wsb, stream=main)
        with self._span("router_bwd_dw"):
            L.moe_grouped_gemm_bwd(x, wr, self.dlogits, self.router_offsets, T, d, E, 1, c,
                                   None, None, self.dwr, ws, wsb, stream=main)
        if overlap:
            main.wait_event(self.ev_side)
        return Grads(self.dx, self.dwr, self.dw1, self.dw2)
