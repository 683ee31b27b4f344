"""Forward and backward of the dropless top-k MoE SwiGLU layer on the GPU.

``MoELayerRunner`` owns the device buffers of one problem size (allocated
through PyTorch, which here only supplies memory and streams) and runs the
layer through the C ABI:

  forward : moe_route_meta (moe_route + moe_permute_meta) -> moe_ffn_gate_up_gather
            (the permute fused into gate/up's row loads) -> moe_permute (the
            grouped copy xs, for the weight gradients) -> moe_ffn_down -> moe_combine
  backward: moe_combine_bwd -> moe_route_bwd -> moe_ffn_bwd_dact ->
            moe_ffn_bwd_dx_dw (dX and the weight gradients) -> moe_permute_bwd
With gather=False gate/up reads xs too (moe_ffn_gate_up).  With
dw_gather=True the weight gradients read the x rows through sorted_flat
(moe_ffn_bwd_dx_dw_gather) and xs is never materialised: NK*H elements less
memory, for a slower weight-gradient launch.  A forward-only runner holds no
xs.

With a shared expert, moe_shared_ffn runs beside the routed path and
moe_combine_shared adds its output; in the backward moe_shared_ffn_bwd gives
its gradients and moe_permute_bwd_add adds its input gradient to dx.

Nothing is read back to the host between the calls.  ``MoEFunction`` wraps
one runner call pair as a ``torch.autograd.Function``.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


class MoELayerRunner:
    """Device buffers and C-ABI calls for fixed (N, H, F, E, K, dtype)."""

    def __init__(self, N: int, H: int, F: int, E: int, K: int, dtype: torch.dtype, device="cuda",
                 backward: bool = True, save_gu: Optional[bool] = None, aux_alpha: Optional[float] = None,
                 capacity: Optional[int] = None, shared_ffn: Optional[int] = None, gather: Optional[bool] = None,
                 dw_gather: bool = False, gemm_tiles: int = L.MOE_TILES_AUTO):
        """aux_alpha: weight of the Switch load-balancing loss; None turns it off.
        capacity: expert capacity (rows per expert, the overflow dropped);
        None is the dropless layer.  shared_ffn: intermediate size Fs of a
        shared expert every token passes through (weights passed to forward
        as ``shared``); None: no shared expert.  gather: gate/up reads the
        grouped rows straight from x; None: whenever N*H < 2^31.  dw_gather:
        the weight gradients read them from x as well, so xs is never
        materialised (needs the gathered gate/up).  gemm_tiles: a
        moe_gemm_tiles value forcing one bf16 GEMM tile family on every
        stage (tests); AUTO lets the library choose per stage."""
        self.N, self.H, self.F, self.E, self.K = N, H, F, E, K
        self.dtype = dtype
        self.device = torch.device(device)
        self.d = L.dims(N, H, F, E, K, L.dtype_code(dtype), gemm_tiles)
        self.capacity = capacity
        self.with_backward = backward
        save_gu = backward if save_gu is None else save_gu
        NK = N * K
        dev = self.device
        i32 = torch.int32
        mt = L.moe_max_tiles(self.d)
        if mt < 0:
            raise L.MoEError("moe_max_tiles", L.MOE_EINVAL)
        self.max_tiles = mt
        # forward buffers
        self.topk = torch.empty((N, K), dtype=i32, device=dev)
        self.gates = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.sorted_flat = torch.empty((NK,), dtype=i32, device=dev)
        self.inv = torch.empty((NK,), dtype=i32, device=dev)
        self.counts = torch.empty((E,), dtype=i32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.tiles = torch.empty((max(1, mt) * 3,), dtype=i32, device=dev)
        self.num_tiles = torch.empty((1,), dtype=i32, device=dev)
        self.meta_ws = self._ws(L.MOE_ENTRY_PERMUTE_META)
        self.route_meta_ws = self._ws(L.MOE_ENTRY_ROUTE_META)
        # the gather is fused into gate/up's row loads; the weight gradients
        # read the grouped copy xs unless dw_gather (then xs never exists)
        fits = N * H < 2 ** 31
        if gather and not fits:
            raise ValueError("gathered row loads need N*H < 2^31")
        self.gather_fused = fits if gather is None else bool(gather)
        if dw_gather and not self.gather_fused:
            raise ValueError("dw_gather needs the gathered gate/up (gather and N*H < 2^31)")
        self.dw_gather = bool(dw_gather) and backward
        need_xs = not self.gather_fused or (backward and not self.dw_gather)
        self.xs = torch.empty((NK, H), dtype=dtype, device=dev) if need_xs else None
        self.g = torch.empty((NK, F), dtype=dtype, device=dev) if save_gu else None
        self.u = torch.empty((NK, F), dtype=dtype, device=dev) if save_gu else None
        self.act = torch.empty((NK, F), dtype=dtype, device=dev)
        self.ys = torch.empty((NK, H), dtype=dtype, device=dev)
        self.y = torch.empty((N, H), dtype=dtype, device=dev)
        self.aux_alpha = aux_alpha
        if aux_alpha is not None:
            self.probs = torch.empty((N, E), dtype=torch.float32, device=dev)
            self.aux_loss = torch.empty((1,), dtype=torch.float32, device=dev)
            self.aux_ws = self._ws(L.MOE_ENTRY_AUX_LOSS)
        if backward:
            f32 = torch.float32
            self.dys = torch.empty((NK, H), dtype=dtype, device=dev)
            self.dgates = torch.empty((N, K), dtype=f32, device=dev)
            self.dlogits = torch.empty((N, E), dtype=f32, device=dev)
            self.dw_r = torch.empty((H, E), dtype=f32, device=dev)
            self.dg = torch.empty((NK, F), dtype=dtype, device=dev)
            self.du = torch.empty((NK, F), dtype=dtype, device=dev)
            self.dxs = torch.empty((NK, H), dtype=dtype, device=dev)
            self.dw_gate = torch.empty((E, H, F), dtype=f32, device=dev)
            self.dw_up = torch.empty((E, H, F), dtype=f32, device=dev)
            self.dw_down = torch.empty((E, F, H), dtype=f32, device=dev)
            self.dx = torch.empty((N, H), dtype=dtype, device=dev)
            self.route_ws = self._ws(L.MOE_ENTRY_ROUTE_BWD if aux_alpha is None else L.MOE_ENTRY_ROUTE_BWD_AUX)
            self.perm_ws = self._ws(L.MOE_ENTRY_PERMUTE_BWD)
        self.shared_ffn = shared_ffn
        if shared_ffn is not None:
            Fs = shared_ffn
            self.ds = L.dims(N, H, Fs, 1, 1, L.dtype_code(dtype))
            self.g_s = torch.empty((N, Fs), dtype=dtype, device=dev) if save_gu else None
            self.u_s = torch.empty((N, Fs), dtype=dtype, device=dev) if save_gu else None
            self.act_s = torch.empty((N, Fs), dtype=dtype, device=dev)
            self.ys_s = torch.empty((N, H), dtype=dtype, device=dev)
            # the backward layout starts with the forward one
            self.shared_ws = self._ws(L.MOE_ENTRY_SHARED_FFN_BWD if backward else L.MOE_ENTRY_SHARED_FFN, self.ds)
            if backward:
                f32 = torch.float32
                self.dg_s = torch.empty((N, Fs), dtype=dtype, device=dev)
                self.du_s = torch.empty((N, Fs), dtype=dtype, device=dev)
                self.dx_s = torch.empty((N, H), dtype=dtype, device=dev)
                self.dw_gate_s = torch.empty((H, Fs), dtype=f32, device=dev)
                self.dw_up_s = torch.empty((H, Fs), dtype=f32, device=dev)
                self.dw_down_s = torch.empty((Fs, H), dtype=f32, device=dev)
        self.inputs = None
        self.shared_w = None

    def _ws(self, entry: int, d=None):
        n = L.moe_workspace_bytes(self.d if d is None else d, entry)
        if n == 2 ** 64 - 1:
            raise L.MoEError("moe_workspace_bytes", L.MOE_EINVAL)
        return torch.empty((max(16, n),), dtype=torch.uint8, device=self.device)

    # -------------------------------------------------------------- forward
    def route(self, x, w_r, bias=None, stream=None):
        L.moe_route(self.d, x, w_r, bias, self.topk, self.gates, stream)

    def meta(self, topk=None, stream=None):
        tk = self.topk if topk is None else topk
        if self.capacity is None:
            L.moe_permute_meta(self.d, tk, self.sorted_flat, self.inv, self.counts, self.offsets, self.tiles,
                               self.num_tiles, self.meta_ws, stream)
        else:
            L.moe_permute_meta_capacity(self.d, tk, self.capacity, self.sorted_flat, self.inv, self.counts,
                                        self.offsets, self.tiles, self.num_tiles, self.meta_ws, stream)

    def forward(self, x, w_r, w_gate, w_up, w_down, bias=None, topk=None, gates=None, stream=None, shared=None,
                side_stream=None):
        """Run the forward; returns y.  ``topk``/``gates`` (optional) replace the
        router's own assignment (moe_route is then skipped).  ``shared`` =
        (W_gate_s [H,Fs], W_up_s [H,Fs], W_down_s [Fs,H]) when the runner has a
        shared expert; with ``side_stream`` it runs there, beside the routed
        path, and the combine waits for it."""
        if (shared is None) != (self.shared_ffn is None):
            raise ValueError("shared weights must be given exactly when the runner has a shared expert")
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        shared_done = None
        if shared is not None:
            side = main if side_stream is None else side_stream
            if side is not main:
                ev = torch.cuda.Event()
                ev.record(main)
                side.wait_event(ev)
            L.moe_shared_ffn(self.ds, x, shared[0], shared[1], shared[2], self.g_s, self.u_s, self.act_s, self.ys_s,
                             self.shared_ws, side)
            if side is not main:
                shared_done = torch.cuda.Event()
                shared_done.record(side)
        stream = main
        if topk is None:
            # router and routing metadata in two launches
            L.moe_route_meta(self.d, x, w_r, bias, 2 ** 31 - 1 if self.capacity is None else self.capacity,
                             self.topk, self.gates, self.sorted_flat, self.inv, self.counts, self.offsets, self.tiles,
                             self.num_tiles, self.route_meta_ws, stream)
        else:
            self.topk.copy_(topk)
            self.gates.copy_(gates)
            self.meta(stream=stream)
        if self.gather_fused:
            L.moe_ffn_gate_up_gather(self.d, x, self.sorted_flat, w_gate, w_up, self.tiles, self.num_tiles, self.g,
                                     self.u, self.act, stream)
            if self.xs is not None:
                L.moe_permute(self.d, x, self.sorted_flat, self.xs, stream)
        else:
            L.moe_permute(self.d, x, self.sorted_flat, self.xs, stream)
            L.moe_ffn_gate_up(self.d, self.xs, w_gate, w_up, self.tiles, self.num_tiles, self.g, self.u, self.act,
                              stream)
        L.moe_ffn_down(self.d, self.act, w_down, self.tiles, self.num_tiles, self.ys, stream)
        if shared is None:
            L.moe_combine(self.d, self.ys, self.gates, self.inv, self.y, stream)
        else:
            if shared_done is not None:
                stream.wait_event(shared_done)
            L.moe_combine_shared(self.d, self.ys, self.gates, self.inv, self.ys_s, self.y, stream)
        if self.aux_alpha is not None:
            L.moe_aux_loss(self.d, x, w_r, bias, self.counts, self.aux_alpha, self.probs, self.aux_loss, self.aux_ws,
                           stream)
        self.inputs = (x, w_r, w_gate, w_up, w_down)
        self.shared_w = shared
        return self.y

    # ------------------------------------------------------------- backward
    def backward(self, dy, stream=None, aux_grad: float = 1.0, side_stream=None):
        """Run the backward of the last forward; returns a dict of gradients.
        aux_grad: upstream gradient of the load-balancing loss (when on).
        side_stream: optional second stream (default priority).  The router
        backward (and the shared expert's backward) then runs beside dA (they
        need only dgates and dy); every launch is
        deterministic by itself, so the results are the same bits either way.
        The grouped GEMMs keep the whole GPU.  ``stream`` waits for the side
        stream before returning."""
        if not self.with_backward:
            raise RuntimeError("runner was built without backward buffers")
        x, w_r, w_gate, w_up, w_down = self.inputs
        d = self.d
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        side = main if side_stream is None else side_stream

        def fork():
            if side is not main:
                ev = torch.cuda.Event()
                ev.record(main)
                side.wait_event(ev)

        def join(into, frm):
            if into is not frm:
                ev = torch.cuda.Event()
                ev.record(frm)
                into.wait_event(ev)

        L.moe_combine_bwd(d, dy, self.ys, self.gates, self.inv, self.dys, self.dgates, main)
        fork()
        if self.aux_alpha is None:
            L.moe_route_bwd(d, x, self.topk, self.gates, self.dgates, self.dlogits, self.dw_r, self.route_ws, side)
        else:
            L.moe_route_bwd_aux(d, x, self.topk, self.gates, self.dgates, self.probs, self.counts,
                                self.aux_alpha * aux_grad, self.dlogits, self.dw_r, self.route_ws, side)
        if self.shared_w is not None:
            # the shared expert's backward needs only dy and its own saved rows
            L.moe_shared_ffn_bwd(self.ds, x, dy, self.shared_w[0], self.shared_w[1], self.shared_w[2], self.g_s,
                                 self.u_s, self.act_s, self.dg_s, self.du_s, self.dx_s, self.dw_gate_s, self.dw_up_s,
                                 self.dw_down_s, self.shared_ws, side)
        route_done = torch.cuda.Event()
        route_done.record(side)
        L.moe_ffn_bwd_dact(d, self.dys, w_down, self.g, self.u, self.tiles, self.num_tiles, self.dg, self.du, main)
        if self.dw_gather:
            L.moe_ffn_bwd_dx_dw_gather(d, self.dg, self.du, w_gate, w_up, self.tiles, self.num_tiles, self.dxs, x,
                                       self.sorted_flat, self.act, self.dys, self.offsets, self.dw_gate, self.dw_up,
                                       self.dw_down, main)
        else:
            L.moe_ffn_bwd_dx_dw(d, self.dg, self.du, w_gate, w_up, self.tiles, self.num_tiles, self.dxs, self.xs,
                                self.act, self.dys, self.offsets, self.dw_gate, self.dw_up, self.dw_down, main)
        if side is not main:
            main.wait_event(route_done)
        if self.shared_w is None:
            permute_bwd = L.moe_permute_bwd if self.aux_alpha is None else L.moe_permute_bwd_dense
            permute_bwd(d, self.dxs, self.inv, self.topk, self.dlogits, w_r, self.dx, self.perm_ws, main)
        else:
            L.moe_permute_bwd_add(d, self.dxs, self.inv, self.topk, self.dlogits, w_r, self.aux_alpha is not None,
                                  self.dx_s, self.dx, self.perm_ws, main)
        join(main, side)
        out = dict(dx=self.dx, dw_r=self.dw_r, dw_gate=self.dw_gate, dw_up=self.dw_up, dw_down=self.dw_down,
                   dgates=self.dgates, dlogits=self.dlogits)
        if self.shared_w is not None:
            out.update(dw_gate_s=self.dw_gate_s, dw_up_s=self.dw_up_s, dw_down_s=self.dw_down_s)
        return out


class MoEFunction(torch.autograd.Function):
    """y = MoE(x) with gradients for x, W_r, W_gate, W_up, W_down and, with a
    shared expert, W_gate_s, W_up_s, W_down_s.

    Weight gradients are computed in float32 by the library and returned in
    the weights' dtype (autograd requires it); use MoELayerRunner directly to
    keep them in float32.  With aux_alpha set, the Switch load-balancing loss
    is returned as a second output that carries no autograd edge: its
    gradient is added to the router's in the backward as if aux_grad * loss
    were part of the training loss (aux_grad is a constant, so no device
    value is read back to the host).
    """

    @staticmethod
    def forward(ctx, x, w_r, w_gate, w_up, w_down, w_gate_s, w_up_s, w_down_s, K: int, bias, capacity, aux_alpha,
                aux_grad, dw_gather):
        N, H = x.shape
        E = w_r.shape[1]
        F = w_gate.shape[2]
        shared = None if w_gate_s is None else (w_gate_s.contiguous(), w_up_s.contiguous(), w_down_s.contiguous())
        r = MoELayerRunner(N, H, F, E, K, x.dtype, x.device, backward=True, aux_alpha=aux_alpha, capacity=capacity,
                           shared_ffn=None if shared is None else shared[0].shape[1], dw_gather=dw_gather)
        y = r.forward(x.contiguous(), w_r.contiguous(), w_gate.contiguous(), w_up.contiguous(), w_down.contiguous(),
                      bias, shared=shared)
        ctx.runner = r
        ctx.aux_grad = aux_grad
        aux = r.aux_loss.clone() if aux_alpha is not None else torch.zeros((1,), dtype=torch.float32,
                                                                             device=x.device)
        ctx.mark_non_differentiable(aux)
        return y.clone(), aux

    @staticmethod
    def backward(ctx, dy, _daux):
        r = ctx.runner
        g = r.backward(dy.contiguous(), aux_grad=ctx.aux_grad)
        cast = lambda t: t.to(r.dtype)
        shared = ((cast(g["dw_gate_s"]), cast(g["dw_up_s"]), cast(g["dw_down_s"])) if r.shared_ffn is not None
                  else (None, None, None))
        return ((g["dx"].clone(), cast(g["dw_r"]), cast(g["dw_gate"]), cast(g["dw_up"]), cast(g["dw_down"])) + shared
                + (None,) * 6)


def moe_layer(x, w_r, w_gate, w_up, w_down, K: int, bias=None, *, capacity: Optional[int] = None,
              shared=None, aux_alpha: Optional[float] = None, aux_grad: float = 1.0, dw_gather: bool = False):
    """Functional form of the layer with autograd support.

    shared = (W_gate_s [H,Fs], W_up_s [H,Fs], W_down_s [Fs,H]) adds a shared
    expert; capacity caps the rows per expert (token dropping); aux_alpha
    turns on the Switch load-balancing loss; dw_gather keeps no grouped copy
    of x for the weight gradients (less memory, slower).  Returns y, or
    (y, aux_loss) when aux_alpha is set.
    """
    ws = (None, None, None) if shared is None else tuple(shared)
    y, aux = MoEFunction.apply(x, w_r, w_gate, w_up, w_down, ws[0], ws[1], ws[2], K, bias, capacity, aux_alpha,
                               aux_grad, dw_gather)
    return (y, aux) if aux_alpha is not None else y
