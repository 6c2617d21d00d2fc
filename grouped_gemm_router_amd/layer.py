"""One MoE expert layer forward on one GPU, as five calls into libmoe.so.

    route -> permute -> grouped GEMM gate/up (+SwiGLU) -> grouped GEMM down
          -> combine

("Dense GEMM to TP MoE" §2.2 data flow; "DeepGEMM walkthrough" §2.1 layer
formula with the shared expert.)  This module only allocates buffers with
torch and passes pointers; every step runs in the library's HIP kernels, on
the current stream, with no host synchronisation and no host round trip of
the per-expert sizes.
"""
from __future__ import annotations

import torch

from . import api


def padded_weights(w: torch.Tensor, pad_bytes: int = 256) -> torch.Tensor:
    """A copy of [G][N][K] weights whose rows sit K + pad_bytes / element size
    elements apart when a row is a power-of-two number of bytes of at least
    4 KB (such rows stream from HBM through few memory channels), else a
    contiguous copy.  The result is a [G][N][K] view that moe_grouped_gemm and
    moe_grouped_gemm_fp8 take as they are.  Measured in the layer: decode-size
    gate/up (8 KB rows) 0.35-0.36 -> 0.33 ms, DeepSeek-shape down (4 KB rows)
    1.93-1.94 -> 1.91 ms, Mixtral shapes unchanged; the 2 KB rows of the
    DeepSeek-shape FP8 down were 2 % slower padded, so they stay dense."""
    G, N, K = w.shape
    row = K * w.element_size()
    if row < 4096 or row & (row - 1):
        return w.contiguous()
    ldb = K + pad_bytes // w.element_size()
    store = torch.empty((G, N, ldb), dtype=w.dtype, device=w.device)
    view = store[:, :, :K]
    view.copy_(w)
    return view


class MoELayer:
    """Weights: w_router [E][d]; w_gate, w_up [G][dff][d]; w_down [G][d][dff]
    with G = E + n_shared (shared experts last), all on the GPU.

    dtype is taken from w_router: fp32 or bf16.  ``fp8=True`` quantises the
    expert weights to E4M3 with 128 x 128 block scales (moe_quantize_fp8) and
    runs both GEMMs in FP8 with 1 x 128 activation scales; the router stays in
    the activation dtype and the output is bf16.
    """

    def __init__(self, w_router, w_gate, w_up, w_down, k, *, n_shared=0, bias=None, fp8=False,
                 renorm=False, keep_logits=True, keep_prob_sums=True, capacity_factor=None):
        self.E, self.d = w_router.shape
        self.G, self.dff, d2 = w_gate.shape
        assert d2 == self.d and self.G == self.E + n_shared
        assert w_up.shape == w_gate.shape and w_down.shape == (self.G, self.d, self.dff)
        self.k, self.n_shared, self.fp8 = k, n_shared, fp8
        self.w_router = w_router.contiguous()
        self.bias = None if bias is None else bias.to(torch.float32).contiguous()
        self.flags = api.MOE_ROUTE_RENORM if renorm else 0
        self.keep_logits = keep_logits
        # per-16-token sums of the gate probabilities, written by the route
        # for router_stats
        self.keep_prob_sums = keep_prob_sums
        # capacity factor cf: each expert keeps at most ceil(cf * T * k / E)
        # routed rows (1.0 = a perfectly even share); None = drop-less
        self.capacity_factor = capacity_factor
        self.act_dtype = w_router.dtype
        self.device = w_router.device
        # expert weights are stored with padded rows where that streams them
        # faster (padded_weights); the GEMMs take the row pitch from the view
        if fp8:
            self.wg_q, self.wg_s = self._quant(w_gate)
            self.wu_q, self.wu_s = self._quant(w_up)
            self.wd_q, self.wd_s = self._quant(w_down)
        else:
            self.w_gate = padded_weights(w_gate)
            self.w_up = padded_weights(w_up)
            self.w_down = padded_weights(w_down)
        self._T = None
        self._gen = 0  # bumped whenever alloc() replaces the buffers
        self._fwd_key, self._fwd_steps = None, None

    def _quant(self, w):
        G, R, Cn = w.shape
        q = torch.empty((G, R, Cn), dtype=torch.uint8, device=self.device)
        s = torch.empty((G, R // 128, Cn // 128), dtype=torch.float32, device=self.device)
        api.moe_quantize_fp8(w.contiguous().view(G * R, Cn), q.view(G * R, Cn),
                             s.view(G * R // 128, Cn // 128), block_rows=128, block_cols=128)
        return padded_weights(q), s

    def capacity(self, T: int):
        """Rows per expert under the capacity factor (None when drop-less)."""
        if self.capacity_factor is None:
            return None
        return int(-(-self.capacity_factor * T * self.k // self.E))

    @property
    def out_dtype(self):
        return torch.bfloat16 if self.fp8 else self.act_dtype

    def alloc(self, T: int):
        """(Re)allocate the intermediate buffers for T tokens."""
        if self._T == T:
            return
        dev, E, k, G, ns = self.device, self.E, self.k, self.G, self.n_shared
        rows = T * k + ns * T
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((T, E), dtype=f32, device=dev) if self.keep_logits else None
        self.prob_sums = (torch.empty((api.prob_sum_blocks(T), E), dtype=f32, device=dev)
                          if self.keep_prob_sums else None)
        self.topk_idx = torch.empty((T, k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=f32, device=dev)
        self.counts = torch.empty((E,), dtype=i32, device=dev)
        self.offsets = torch.empty((G + 1,), dtype=i32, device=dev)
        self.perm_src = torch.empty((T * k,), dtype=i32, device=dev)
        self.flat_to_row = torch.empty((T * k + ns * T,), dtype=i32, device=dev)
        if self.capacity_factor is not None:
            self.overflow = torch.empty((T * k,), dtype=i32, device=dev)
            self.n_overflow = torch.empty((1,), dtype=i32, device=dev)
        # route, permute and the two GEMMs run one after the other on one
        # stream, so they share one workspace
        ws = max(api.moe_permute_workspace_size(T, k, E),
                 api.moe_route_workspace_size(T, self.d, E))
        if not self.fp8:
            ws = max(ws,
                     api.moe_grouped_gemm_workspace_size(G, rows, self.dff, self.d,
                                                         self.act_dtype, api.MOE_EPI_SWIGLU),
                     api.moe_grouped_gemm_workspace_size(G, rows, self.d, self.dff,
                                                         self.act_dtype, api.MOE_EPI_NONE))
        self.ws = torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev)
        if self.fp8:
            self.x_perm = torch.empty((rows, self.d), dtype=torch.uint8, device=dev)
            # scales group-major, [columns/128][rows]
            self.x_scale = torch.empty((self.d // 128, rows), dtype=f32, device=dev)
            self.h = torch.empty((rows, self.dff), dtype=torch.uint8, device=dev)
            self.h_scale = torch.empty((self.dff // 128, rows), dtype=f32, device=dev)
            self.y = torch.empty((rows, self.d), dtype=torch.bfloat16, device=dev)
        else:
            self.x_perm = torch.empty((rows, self.d), dtype=self.act_dtype, device=dev)
            self.x_scale = None
            self.h = torch.empty((rows, self.dff), dtype=self.act_dtype, device=dev)
            self.h_scale = None
            # expert outputs stay fp32 until the combine: a bf16 Y plus a bf16
            # out would be two roundings of the largest outputs
            self.y = torch.empty((rows, self.d), dtype=torch.float32, device=dev)
        self._T = T
        self._gen += 1

    def steps(self, x, out):
        """The five calls on x -> out, as (name, thunk) pairs (for timing each
        one): marshalled once here, on the current stream, so a thunk costs
        one ctypes call.  They stay valid while the layer's buffers do (the
        next alloc() with another T replaces them)."""
        ns = self.n_shared
        d = api.deferred
        s = [("route", d(api.moe_route, x, self.w_router, self.topk_idx, self.topk_w,
                         logits=self.logits, logit_bias=self.bias, flags=self.flags,
                         prob_sums=self.prob_sums, ws=self.ws)),
             ("permute", self._permute_fn(x))]
        if self.fp8:
            s.append(("gemm_gate_up", d(
                api.moe_grouped_gemm_fp8, self.x_perm, self.x_scale, self.wg_q, self.wg_s, self.h,
                self.offsets, B2_q=self.wu_q, B2_scale=self.wu_s, C_scale=self.h_scale,
                epi=api.MOE_EPI_SWIGLU)))
            s.append(("gemm_down", d(api.moe_grouped_gemm_fp8, self.h, self.h_scale, self.wd_q,
                                     self.wd_s, self.y, self.offsets)))
        else:
            s.append(("gemm_gate_up", d(api.moe_grouped_gemm, self.x_perm, self.w_gate, self.h,
                                        self.offsets, B2=self.w_up, epi=api.MOE_EPI_SWIGLU,
                                        ws=self.ws)))
            s.append(("gemm_down", d(api.moe_grouped_gemm, self.h, self.w_down, self.y,
                                     self.offsets, ws=self.ws)))
        s.append(("combine", d(api.moe_combine, self.y, self.flat_to_row, self.topk_w, out,
                               n_shared=ns)))
        return s

    def _permute_fn(self, x):
        E, ns = self.E, self.n_shared
        cap = self.capacity(x.shape[0])
        if cap is None:
            return api.deferred(api.moe_permute, x, self.topk_idx, E, ns, self.x_perm,
                                self.counts, self.offsets, self.perm_src, self.flat_to_row,
                                self.ws, x_perm_scale=self.x_scale)
        return api.deferred(api.moe_permute_capped, x, self.topk_idx, E, ns, cap, self.x_perm,
                            self.counts, self.offsets, self.perm_src, self.flat_to_row, self.ws,
                            overflow=self.overflow, n_overflow=self.n_overflow,
                            x_perm_scale=self.x_scale)

    def router_stats(self, alpha: float = 0.01):
        """Load-balance statistics of the last forward (needs keep_prob_sums):
        f [E], P [E] and summary [3] = (aux loss, max/mean, entropy bits),
        as device tensors, enqueued on the current stream (one launch over
        the route's probability sums and the permute's counts)."""
        if self.prob_sums is None:
            raise RuntimeError("router_stats needs the route's probability sums: build the "
                               "layer with keep_prob_sums=True")
        T = self._T
        f = torch.empty((self.E,), dtype=torch.float32, device=self.device)
        P = torch.empty_like(f)
        summary = torch.empty((3,), dtype=torch.float32, device=self.device)
        api.moe_router_stats(self.prob_sums, self.counts, T, self.k, alpha, f, P, summary)
        return {"f": f, "P": P, "aux_loss": summary[0], "max_over_mean": summary[1],
                "entropy_bits": summary[2]}

    def capture(self, x, out):
        """A HIP graph (torch.cuda.CUDAGraph) of the five calls on x -> out,
        for callers that run the same shapes again and again: one replay
        launches the whole layer without the host-side cost of five library
        calls.  The buffers are allocated before the capture; none of the
        library's kernels needs a memset, so the graph holds kernel nodes
        only.  Replaying it recomputes out from the current contents of x."""
        T = x.shape[0]
        assert out.shape == (T, self.d) and out.dtype == self.out_dtype
        self.alloc(T)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager pass before the capture
            for _, fn in self.steps(x, out):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _, fn in self.steps(x, out):
                fn()
        return g

    def forward(self, x, out=None):
        T, d = x.shape
        assert d == self.d and x.dtype == self.act_dtype and x.is_contiguous()
        self.alloc(T)
        if out is None:
            out = torch.empty((T, d), dtype=self.out_dtype, device=self.device)
        # the marshalled calls are kept while x, out, the stream and the
        # buffers stay the same (a serving loop that reuses its tensors); they
        # hold the last x and out until then
        key = (x.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream,
               self._gen)
        if key != self._fwd_key:
            self._fwd_steps, self._fwd_key = self.steps(x, out), key
        for _, fn in self._fwd_steps:
            fn()
        return out

    __call__ = forward
