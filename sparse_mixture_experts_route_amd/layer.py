"""Layer-level wrapper over the C-ABI: buffer allocation (torch, device
memory only), the call sequence route -> dispatch -> (aux loss) ->
ffn_forward, the backward call, and the deferred balance state machine.

The deferred balance follows "Sparse MoE FFN for DFlash-family drafters"
(What's here: a training forward stashes its routing counts; the next forward
applies them to the fp32 bias before routing, outside any recompute region;
eval forwards stash nothing; a second apply is a no-op).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import _lib as L


@dataclass
class RouterState:
    """State a stateful router threads from one call to the next
    ("mstar.model.components.moe", Router contract: router_states in,
    router_states_next out): the fp32 selection bias and the expert loads of
    the last training forward that are not yet applied to it (None when
    nothing is pending)."""
    bias: torch.Tensor
    counts: Optional[torch.Tensor] = None
    tokens_k: int = 0


class BalanceController:
    """fp32 selection bias plus the stash of the last training forward's
    expert counts (device tensors, so no host sync)."""

    def __init__(self, bias: torch.Tensor, rate: float):
        assert bias.dtype == torch.float32
        self.bias = bias
        self.rate = float(rate)
        self.stash = torch.zeros(bias.shape[0], dtype=torch.int32, device=bias.device)
        self.pending = False
        self.stash_tokens_k = 0

    def apply_pending(self, shape: L.MoeShape) -> bool:
        if not self.pending:
            return False
        sh = L.MoeShape(*[getattr(shape, f) for f, _ in L.MoeShape._fields_])
        sh.T = self.stash_tokens_k // sh.k
        L.moe_balance_counts(sh, None, self.stash, self.bias, self.rate)
        self.pending = False
        return True

    def after_forward(self, counts: torch.Tensor, tokens_k: int, training: bool) -> None:
        if training:
            self.stash.copy_(counts)
            self.stash_tokens_k = int(tokens_k)
            self.pending = True


class MoEFFN:
    """Sparse MoE FFN layer on one device.

    params: w_router [E,H], w_gate_up [E,2I,H], w_down [E,H,I], and
    optionally ws_gate_up [2Is,H], ws_down [H,Is], w_shared_gate [H].
    aux_alpha > 0: a training forward also computes the load-balancing aux
    loss (``last["aux_loss"]``, a [1] fp32 device tensor) and the backward
    differentiates sum(out * dout) + aux_loss."""

    def __init__(self, shape: L.MoeShape, params: Dict[str, torch.Tensor],
                 sel_bias: Optional[torch.Tensor] = None, rate: float = 1e-3,
                 fuse_gather: bool = True, aux_alpha: float = 0.0):
        self.shape = shape
        self.p = params
        self.aux_alpha = float(aux_alpha)
        self.balance = BalanceController(sel_bias, rate) if sel_bias is not None else None
        self.fuse_gather = fuse_gather
        self.weights = L.weights_struct(params["w_gate_up"], params["w_down"], params.get("ws_gate_up"),
                                        params.get("ws_down"), params.get("w_shared_gate"))
        self._ws: Dict[int, torch.Tensor] = {}
        self.last: Dict[str, torch.Tensor] = {}

    def _shape_T(self, T: int) -> L.MoeShape:
        sh = L.MoeShape(*[getattr(self.shape, f) for f, _ in L.MoeShape._fields_])
        sh.T = T
        return sh

    def _workspace(self, sh: L.MoeShape, op: int, device) -> torch.Tensor:
        need = L.workspace_bytes(sh, op)
        cur = self._ws.get(op)
        if cur is None or cur.numel() < need:
            cur = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
            self._ws[op] = cur
        return cur

    def route(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
              router_states: Optional[RouterState] = None):
        """Router contract: (tokens, hidden) -> (weights (tokens,k) fp32,
        ids (tokens,k) int64, router_states_next).  Without a selection bias
        the router is stateless: router_states is ignored and the returned
        state is None.  With one it is stateful: it routes with the bias of
        router_states after applying the loads it carries (or with the
        layer's own state when router_states is None) and returns that bias
        with nothing pending (routing alone stashes no loads)."""
        if self.balance is None:
            out = self._route(x, logits_out=logits)
            return out["weights"], out["ids"], None
        if router_states is None:
            router_states = self.router_state()
        bias = self._applied_bias(router_states, x.shape[0])
        out = self._route(x, logits_out=logits, bias=bias)
        return out["weights"], out["ids"], RouterState(bias)

    def router_state(self) -> Optional[RouterState]:
        """The layer's own router state (None for a stateless router)."""
        if self.balance is None:
            return None
        b = self.balance
        return RouterState(b.bias, b.stash if b.pending else None, b.stash_tokens_k if b.pending else 0)

    def _applied_bias(self, st: RouterState, T: int) -> torch.Tensor:
        """st.bias with st.counts applied (a new tensor when counts are
        pending; st itself is left unchanged)."""
        if st.counts is None:
            return st.bias
        bias = st.bias.clone()
        sh = self._shape_T(st.tokens_k // self.shape.k)
        L.moe_balance_counts(sh, None, st.counts, bias, self.balance.rate)
        return bias

    def _route(self, x, logits_out=None, want_logits=False, want_sums=False, bias=None, dispatch=False):
        """moe_route; with dispatch, moe_route_dispatch (the expert counts,
        segment offsets and the permutation come with the routing)."""
        sh = self._shape_T(x.shape[0])
        dev = x.device
        T, E, k = sh.T, sh.E, sh.k
        weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int64, device=dev)
        logits = logits_out
        if logits is None and want_logits:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        gate = None
        if sh.Is and sh.shared_gated:
            gate = torch.empty((T,), dtype=torch.float32, device=dev)
        if bias is None and self.balance is not None:
            bias = self.balance.bias
        sums = torch.empty((E,), dtype=torch.float32, device=dev) if want_sums else None
        wg = self.p.get("w_shared_gate") if gate is not None else None
        out = {"weights": weights, "ids": ids, "logits": logits, "gate": gate, "score_sums": sums}
        if dispatch:
            P = T * k
            d = {"counts": torch.empty((E,), dtype=torch.int32, device=dev),
                 "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
                 "perm": torch.empty((P,), dtype=torch.int32, device=dev),
                 "pos": torch.empty((P,), dtype=torch.int32, device=dev)}
            L.moe_route_dispatch(sh, x, self.p["w_router"], wg, bias, logits, weights, ids, gate, d["counts"],
                                 d["offsets"], d["perm"], d["pos"], self._workspace(sh, L.OP_ROUTE_DISPATCH, dev),
                                 score_sums=sums)
            return {**out, **d}
        # scratch of the score sums and of the split reduction short batches take
        ws = self._workspace(sh, L.OP_ROUTE, dev)
        L.moe_route(sh, x, self.p["w_router"], wg, bias, logits, weights, ids, gate, score_sums=sums, ws=ws)
        return out

    def _forward_whole(self, x, bias, out):
        """moe_layer_forward: routing, sort, experts and combine in one call
        (outputs as moe_route_dispatch's and moe_ffn_forward's)."""
        sh = self._shape_T(x.shape[0])
        dev = x.device
        T, E, k = sh.T, sh.E, sh.k
        P = T * k
        gate = torch.empty((T,), dtype=torch.float32, device=dev) if (sh.Is and sh.shared_gated) else None
        if bias is None and self.balance is not None:
            bias = self.balance.bias
        r = {"weights": torch.empty((T, k), dtype=torch.float32, device=dev),
             "ids": torch.empty((T, k), dtype=torch.int64, device=dev), "logits": None, "gate": gate,
             "score_sums": None, "counts": torch.empty((E,), dtype=torch.int32, device=dev),
             "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
             "perm": torch.empty((P,), dtype=torch.int32, device=dev),
             "pos": torch.empty((P,), dtype=torch.int32, device=dev)}
        wg = self.p.get("w_shared_gate") if gate is not None else None
        L.moe_layer_forward(sh, self.weights, x, self.p["w_router"], wg, bias, r["weights"], r["ids"], gate,
                            r["counts"], r["offsets"], r["perm"], r["pos"], out,
                            self._workspace(sh, L.OP_LAYER_FORWARD, dev))
        return r

    def forward(self, x: torch.Tensor, training: bool = False, save: bool = False,
                router_states: Optional[RouterState] = None, return_router_states: bool = False):
        """The layer output [T,H].  router_states (stateful router only):
        route with that state instead of the layer's own, which is then left
        untouched.  return_router_states: also return router_states_next,
        the bias used by this call plus, for a training forward, this call's
        loads pending for the next one (None for a stateless router)."""
        sh = self._shape_T(x.shape[0])
        bias = None
        if self.balance is not None:
            if router_states is None:
                self.balance.apply_pending(sh)
            else:
                bias = self._applied_bias(router_states, x.shape[0])
        dev = x.device
        T, H, E, k, I, Is = sh.T, sh.H, sh.E, sh.k, sh.I, sh.Is
        P = T * k
        aux = training and self.aux_alpha != 0.0 and T > 0
        x_sorted = None
        whole = self.fuse_gather and not save and not aux  # the inference forward as one library call
        if whole:
            out = torch.empty_like(x)
            r = self._forward_whole(x, bias, out)
            counts, offsets, perm, pos = r["counts"], r["offsets"], r["perm"], r["pos"]
        elif self.fuse_gather:  # rows read through perm by the gate_up GEMM: routing and sort in one call
            r = self._route(x, want_logits=save, want_sums=aux, bias=bias, dispatch=True)
            counts, offsets, perm, pos = r["counts"], r["offsets"], r["perm"], r["pos"]
        else:                 # the sort with a gathered copy of the rows
            r = self._route(x, want_logits=save, want_sums=aux, bias=bias)
            counts = torch.empty((E,), dtype=torch.int32, device=dev)
            offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
            perm = torch.empty((P,), dtype=torch.int32, device=dev)
            pos = torch.empty((P,), dtype=torch.int32, device=dev)
            x_sorted = torch.empty((P, H), dtype=x.dtype, device=dev)
            L.moe_dispatch(sh, r["ids"], x, counts, offsets, perm, pos, x_sorted,
                           self._workspace(sh, L.OP_DISPATCH, dev))
        aux_out = {}
        if aux:
            aux_out = {"aux_loss": torch.empty((1,), dtype=torch.float32, device=dev),
                       "aux_coef": torch.empty((E,), dtype=torch.float32, device=dev)}
            L.moe_aux_loss(sh, r["score_sums"], counts, self.aux_alpha, aux_out["aux_loss"], aux_out["aux_coef"])
        saved = None
        st = {}
        if save:
            # expert outputs y, s_y: binary16 in a bf16 layer, fp32 in an fp32 one
            ydt = torch.float16 if x.dtype == torch.bfloat16 else torch.float32
            st = {"gu": torch.empty((P, 2 * I), dtype=torch.float32, device=dev),
                  "h": torch.empty((P, I), dtype=x.dtype, device=dev),
                  "y": torch.empty((P, H), dtype=ydt, device=dev)}
            if Is:
                st.update({"s_gu": torch.empty((T, 2 * Is), dtype=torch.float32, device=dev),
                           "s_h": torch.empty((T, Is), dtype=x.dtype, device=dev),
                           "s_y": torch.empty((T, H), dtype=ydt, device=dev)})
            saved = L.saved_struct(**st)
        if not whole:
            out = torch.empty_like(x)
            L.moe_ffn_forward(sh, self.weights, x, x_sorted, offsets, perm, pos, r["weights"], r["gate"], out,
                              saved, self._workspace(sh, L.OP_FFN_FORWARD, dev))
        state_next = None
        if self.balance is not None:
            if router_states is None:
                self.balance.after_forward(counts, P, training)
                state_next = self.router_state()
            else:
                state_next = RouterState(bias, counts if training else None, P if training else 0)
        self.last = {"x": x, "x_sorted": x_sorted, "counts": counts, "offsets": offsets, "perm": perm,
                     "pos": pos, "out": out, **r, **st, **aux_out}
        return (out, state_next) if return_router_states else out

    def backward(self, dout: torch.Tensor, want_dlogits: bool = False) -> Dict[str, torch.Tensor]:
        """Gradients for the last forward (which must have run with save=True)."""
        s = self.last
        x = s["x"]
        sh = self._shape_T(x.shape[0])
        dev = x.device
        T, H, E, I, Is = sh.T, sh.H, sh.E, sh.I, sh.Is
        f32 = torch.float32

        def wgrad(name):  # weight gradients are fp32
            return torch.empty(self.p[name].shape, dtype=f32, device=dev)
        g = {"dx": torch.empty_like(x), "dw_router": wgrad("w_router"), "dw_gate_up": wgrad("w_gate_up"),
             "dw_down": wgrad("w_down")}
        if Is:
            g["dws_gate_up"] = wgrad("ws_gate_up")
            g["dws_down"] = wgrad("ws_down")
            if sh.shared_gated:
                g["dw_shared_gate"] = wgrad("w_shared_gate")
        if want_dlogits:
            g["dlogits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
        saved = L.saved_struct(s["gu"], s["h"], s["y"], s.get("s_gu"), s.get("s_h"), s.get("s_y"))
        L.moe_ffn_backward(sh, self.weights, x, self.p["w_router"], s["logits"], s["ids"], s["weights"],
                           s["gate"], s["offsets"], s["perm"], s["pos"], s["x_sorted"], saved, dout,
                           L.grads_struct(**g), self._workspace(sh, L.OP_FFN_BACKWARD, dev),
                           aux_coef=s.get("aux_coef"))
        return g


def tp_share_params(params: Dict[str, torch.Tensor], n: int, r: int) -> Dict[str, torch.Tensor]:
    """Expert weights of share r of an n-way tensor-parallel split
    ("mstar.model.components.moe", ParallelSparseMoeBlock: expert weights are
    split along the intermediate dimension): the r-th I/n slice of the gate
    rows and of the up rows of every w_gate_up[e] (stacked gate then up, as
    in the full layout), the matching columns of w_down, and the same for the
    shared expert with Is/n.  Returns contiguous copies; the router and the
    shared gate stay whole (every share routes identically)."""
    wgu = params["w_gate_up"]
    I = wgu.shape[1] // 2
    assert I % n == 0
    a, b = r * (I // n), (r + 1) * (I // n)
    out = {"w_gate_up": torch.cat([wgu[:, a:b], wgu[:, I + a:I + b]], dim=1).contiguous(),
           "w_down": params["w_down"][:, :, a:b].contiguous()}
    if "ws_gate_up" in params:
        wsgu = params["ws_gate_up"]
        Is = wsgu.shape[0] // 2
        assert Is % n == 0
        a, b = r * (Is // n), (r + 1) * (Is // n)
        out["ws_gate_up"] = torch.cat([wsgu[a:b], wsgu[Is + a:Is + b]], dim=0).contiguous()
        out["ws_down"] = params["ws_down"][:, a:b].contiguous()
    return out


def forward_partial(shape: L.MoeShape, share: Dict[str, torch.Tensor], n: int, x: torch.Tensor,
                    offsets: torch.Tensor, perm: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """One share's pre-top-k-sum partials (y_part [T*k,H] fp32 sorted rows,
    s_part [T,H] fp32 or None) for the routing of the whole layer."""
    sh = L.MoeShape(*[getattr(shape, f) for f, _ in L.MoeShape._fields_])
    sh.T = x.shape[0]
    sh.I, sh.Is = shape.I // n, shape.Is // n
    dev = x.device
    y = torch.empty((sh.T * sh.k, sh.H), dtype=torch.float32, device=dev)
    sy = torch.empty((sh.T, sh.H), dtype=torch.float32, device=dev) if sh.Is else None
    need = max(L.workspace_bytes(sh, L.OP_FFN_PARTIAL), 256)
    if ws is None or ws.numel() < need:
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    wst = L.weights_struct(share["w_gate_up"], share["w_down"], share.get("ws_gate_up"), share.get("ws_down"))
    L.moe_ffn_forward_partial(sh, wst, x, None, offsets, perm, y, sy, None, ws)
    return y, sy


class ParallelDenseMoEBlock:
    """A dense MLP and the MoE side by side (the DeepSpec issue "Feat:
    Compatible with Gamme4 MoE structure", Decoder layer forward pass): the
    router reads the residual stream, the experts read its RMS-normalised
    copy, the two outputs are normalised, summed, normalised again, added to
    the residual and scaled by the layer scalar.

    moe: the MoEFFN whose router and experts form the MoE branch (built
    without a shared expert); dense: {"w_gate_up" [2Id,H], "w_down" [H,Id]};
    norms: {"g_pre_moe", "g_post_dense", "g_post_moe", "g_post"} [H] each, in
    the layer dtype, applied as given."""

    def __init__(self, moe: MoEFFN, dense: Dict[str, torch.Tensor], norms: Dict[str, torch.Tensor],
                 eps: float = 1e-6, layer_scalar: float = 1.0):
        assert moe.shape.Is == 0, "the dense MLP takes the shared-expert slots of the block"
        self.moe = moe
        self.dense = dense
        self.norms = norms
        self.eps = float(eps)
        self.layer_scalar = float(layer_scalar)
        sh = L.MoeShape(*[getattr(moe.shape, f) for f, _ in L.MoeShape._fields_])
        sh.Is = dense["w_down"].shape[1]
        self.shape = sh
        self.weights = L.weights_struct(moe.p["w_gate_up"], moe.p["w_down"], dense["w_gate_up"], dense["w_down"])
        self._ws: Optional[torch.Tensor] = None

    def forward(self, residual: torch.Tensor, x_dense: torch.Tensor) -> torch.Tensor:
        m = self.moe
        T = residual.shape[0]
        if m.balance is not None:
            m.balance.apply_pending(m._shape_T(T))
        r = m._route(residual, dispatch=True)       # the router reads the residual
        sh = m._shape_T(T)
        dev = residual.device
        counts, offsets, perm, pos = r["counts"], r["offsets"], r["perm"], r["pos"]
        bsh = L.MoeShape(*[getattr(self.shape, f) for f, _ in L.MoeShape._fields_])
        bsh.T = T
        need = max(L.workspace_bytes(bsh, L.OP_BLOCK), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        n = self.norms
        norms = L.block_norms(n["g_pre_moe"], n["g_post_dense"], n["g_post_moe"], n["g_post"], self.eps,
                              self.layer_scalar)
        out = torch.empty_like(residual)
        L.moe_parallel_block_forward(bsh, self.weights, norms, residual, x_dense, offsets, perm, pos, r["weights"],
                                     out, self._ws)
        m.last = {"out": out, **r}
        return out
