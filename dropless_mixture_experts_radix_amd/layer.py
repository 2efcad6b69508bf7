"""A dropless MoE layer on one GPU: buffers plus the four C-ABI calls.

torch provides the device memory and the stream; every step of the layer runs
in the HIP library (route -> permute -> grouped MLP -> combine).
"""
import torch

from . import _lib as M


class MoELayer:
    """Holds prepared weights and the per-call buffers of one layer shape.

    T, H, E, K, F: tokens, hidden, experts seen by the router, routes per token,
    expert FFN width.  L local experts e0..e0+L-1 (default: all).  dtype: the
    expert path (M.F32, M.BF16, M.MXFP8 or M.MXFP4); x_dtype: the token rows (M.F32 or
    M.BF16).  w_router [H,E] (fp32 or bf16) enables the fused projection; when
    it is None, forward() takes logits.
    """

    def __init__(self, T, H, E, K, F, dtype, x_dtype, *, L=None, e0=0, score=M.SOFTMAX, w_router=None,
                 bias=None, capacity=None, device="cuda"):
        self.T, self.H, self.E, self.K, self.F = T, H, E, K, F
        self.L = E if L is None else L
        self.e0, self.score, self.dtype, self.x_dtype = e0, score, dtype, x_dtype
        self.device = torch.device(device)
        sizes = M.moe_query_sizes(T, H, E, K, F, dtype, x_dtype=x_dtype,
                                  w_dtype=M.dtype_code(w_router.dtype) if w_router is not None else M.F32,
                                  L=self.L)
        self.capacity = sizes["capacity"] if capacity is None else capacity
        dev = self.device
        L, cap = self.L, self.capacity
        self.bias = bias
        self.w_dtype = M.F32
        self.w_prep = None
        if w_router is not None:
            self.w_dtype = M.dtype_code(w_router.dtype)
            nb = M.moe_router_prepared_bytes(H, E, self.w_dtype, x_dtype)
            self.w_prep = torch.empty(nb, dtype=torch.uint8, device=dev)
            M.moe_prepare_router(w_router, x_dtype, self.w_prep)
        mx = dtype in (M.MXFP8, M.MXFP4)
        wdt = torch.uint8 if mx else {M.F32: torch.float32, M.BF16: torch.bfloat16}[dtype]
        # bf16 and MX prepared weights come in whole 256-row panels (k-blocked);
        # MXFP4 codes are two per byte
        pad = (lambda n: (n + 255) // 256 * 256) if dtype != M.F32 else (lambda n: n)
        cw = (lambda n: n // 2) if dtype == M.MXFP4 else (lambda n: n)
        self.w1p = torch.empty((L, pad(2 * F), cw(H)), dtype=wdt, device=dev)
        self.w2p = torch.empty((L, pad(H), cw(F)), dtype=wdt, device=dev)
        self.w1s = self.w2s = None
        if mx:
            # E8M0 scales: 16 bytes per prepared row and 512-wide k group
            self.w1s = torch.empty((L, pad(2 * F), (H + 511) // 512 * 16), dtype=torch.uint8, device=dev)
            self.w2s = torch.empty((L, pad(H), (F + 511) // 512 * 16), dtype=torch.uint8, device=dev)
        # per-call buffers
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((T, K), dtype=torch.int16, device=dev)
        self.probs = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.logits_out = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.route_ws = torch.empty(max(M.moe_route_workspace_bytes(T, E, H, x_dtype), 256), dtype=torch.uint8,
                                    device=dev)
        self.counts = torch.empty(L, **i32)
        self.offsets = torch.empty(L + 1, **i32)
        act = torch.float32 if dtype == M.F32 else torch.bfloat16
        self.out_dtype = act
        self.x_perm = torch.empty((cap, cw(H)), dtype=torch.uint8 if mx else act, device=dev)
        self.x_perm_scales = torch.empty((cap, H // 32), dtype=torch.uint8, device=dev) if mx else None
        self.row_to_slot = torch.empty(cap, **i32)
        self.slot_to_row = torch.empty((T, K), **i32)
        # zero-filled once: the permute's state (counter, tile counts) starts and is left at zero
        self.perm_ws = torch.zeros(M.moe_permute_workspace_bytes(T, K, L), dtype=torch.uint8, device=dev)
        self.y_perm = torch.empty((cap, H), dtype=act, device=dev)
        self.mlp_ws = torch.empty(M.moe_grouped_mlp_workspace_bytes(cap, F, dtype), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=act, device=dev)
        self.err = torch.zeros(1, **i32)

    # ------------------------------------------------------------------ weights
    def set_expert_weights(self, e, w1, w2):
        """Prepare local expert e from its logical weights W1 [H,2F], W2 [F,H] (on the GPU)."""
        M.moe_prepare_weights(w1.unsqueeze(0), w2.unsqueeze(0), self.dtype, self.w1p[e:e + 1], self.w2p[e:e + 1],
                              None if self.w1s is None else self.w1s[e:e + 1],
                              None if self.w2s is None else self.w2s[e:e + 1])

    def activations(self):
        """The intermediate `a` of the grouped MLP as stored in its workspace."""
        cap, F = self.capacity, self.F
        if self.dtype == M.F32:
            return self.mlp_ws[: cap * F * 4].view(torch.float32).view(cap, F)
        if self.dtype == M.BF16:  # k-blocked [F/32][capacity][32]
            blk = self.mlp_ws[: cap * F * 2].view(torch.bfloat16).view(F // 32, cap, 32)
            return blk.permute(1, 0, 2).reshape(cap, F)
        cb = F // 2 if self.dtype == M.MXFP4 else F  # code bytes per row
        codes = self.mlp_ws[: cap * cb].view(cap, cb)
        off = (cap * cb + 255) // 256 * 256
        scales = self.mlp_ws[off: off + cap * (F // 32)].view(cap, F // 32)
        return codes, scales

    # ------------------------------------------------------------------ stages
    def route(self, x=None, logits=None, mask=None, write_logits=False):
        M.moe_route_topk(self.ids, self.probs, self.score, logits=logits, x=x, w_prepared=self.w_prep,
                         w_dtype=self.w_dtype, E=self.E, bias=self.bias, mask=mask,
                         logits_out=self.logits_out if write_logits else None, err=self.err,
                         workspace=self.route_ws)

    def permute(self, x):
        M.moe_permute(x, self.ids, self.E, self.e0, self.L, self.counts, self.offsets, self.x_perm,
                      self.row_to_slot, self.slot_to_row, self.perm_ws, x_perm_scales=self.x_perm_scales,
                      err=self.err, out_dtype=self.dtype)

    def mlp(self):
        M.moe_grouped_mlp(self.x_perm, self.offsets, self.w1p, self.w2p, self.y_perm, self.mlp_ws, self.dtype,
                          self.H, self.F, x_perm_scales=self.x_perm_scales, w1p_scales=self.w1s,
                          w2p_scales=self.w2s)

    def combine(self):
        M.moe_unpermute_combine(self.y_perm, self.slot_to_row, self.probs, self.out)

    def forward(self, x, logits=None, mask=None, write_logits=False):
        self.route(x=None if logits is not None else x, logits=logits, mask=mask, write_logits=write_logits)
        self.permute(x)
        self.mlp()
        self.combine()
        return self.out
