"""ctypes binding of libmoe_mi355x.so.  Argument marshalling only: every
step of the layer runs in the library's HIP kernels.  The functions take
torch tensors on the current HIP device and enqueue on torch's current
stream.  Loading fails loudly when the library is missing."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_ELAUNCH = 0, -1, -2, -3, -4
SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_SQRTSOFTPLUS = 0, 1, 2
DTYPE_FP32, DTYPE_BF16 = 0, 1
ROUTE_LOGITS_IN = 1
OP_DISPATCH, OP_FFN_FORWARD, OP_FFN_BACKWARD, OP_ROUTE, OP_FFN_PARTIAL, OP_BLOCK, OP_ROUTE_DISPATCH = 1, 2, 3, 4, 5, 6, 7
OP_LAYER_FORWARD = 8

EXPORTED = ("moe_route", "moe_dispatch", "moe_route_dispatch", "moe_ffn_forward", "moe_layer_forward",
            "moe_ffn_forward_noalloc", "moe_ffn_forward_partial",
            "moe_combine",
            "moe_parallel_block_forward", "moe_ffn_backward", "moe_aux_loss",
            "moe_balance_counts", "moe_score_f32", "moe_bandwidth_probe", "moe_profile_begin",
            "moe_profile_end", "moe_workspace_bytes", "moe_status_str")
N_STAGES = 13
STAGE_NAMES = ("gate_up", "down", "shared_gate_up", "shared_down", "combine", "combine_bwd", "dgrad_dh",
               "wgrad_down", "wgrad_gate_up", "dgrad_dx", "shared_bwd", "router_bwd", "dx_sum")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("I", ctypes.c_int64), ("Is", ctypes.c_int64),
                ("score", ctypes.c_int32), ("renorm", ctypes.c_int32),
                ("shared_gated", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("ws_gate_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
                ("w_shared_gate", ctypes.c_void_p)]


class MoeSaved(ctypes.Structure):
    _fields_ = [("gu", ctypes.c_void_p), ("h", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("s_gu", ctypes.c_void_p), ("s_h", ctypes.c_void_p), ("s_y", ctypes.c_void_p)]


class MoeGrads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dw_router", ctypes.c_void_p),
                ("dw_gate_up", ctypes.c_void_p), ("dw_down", ctypes.c_void_p),
                ("dws_gate_up", ctypes.c_void_p), ("dws_down", ctypes.c_void_p),
                ("dw_shared_gate", ctypes.c_void_p), ("dlogits", ctypes.c_void_p)]


class MoeBlockNorms(ctypes.Structure):
    _fields_ = [("g_pre_moe", ctypes.c_void_p), ("g_post_dense", ctypes.c_void_p),
                ("g_post_moe", ctypes.c_void_p), ("g_post", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("layer_scalar", ctypes.c_float)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mixture_experts_route_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    lib.moe_route.argtypes = [P(MoeShape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, vp]
    lib.moe_aux_loss.argtypes = [P(MoeShape), vp, vp, ctypes.c_float, vp, vp, vp]
    lib.moe_dispatch.argtypes = [P(MoeShape), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_dispatch.argtypes = [P(MoeShape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       i32, vp]
    lib.moe_ffn_forward.argtypes = [P(MoeShape), P(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp,
                                    P(MoeSaved), vp, sz, vp]
    lib.moe_layer_forward.argtypes = [P(MoeShape), P(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.moe_ffn_forward_noalloc.argtypes = [P(MoeShape), P(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_ffn_forward_partial.argtypes = [P(MoeShape), P(MoeWeights), vp, vp, vp, vp, vp, vp, P(MoeSaved),
                                            vp, sz, vp]
    lib.moe_combine.argtypes = [P(MoeShape), vp, vp, vp, vp, vp, vp, vp]
    lib.moe_parallel_block_forward.argtypes = [P(MoeShape), P(MoeWeights), P(MoeBlockNorms), vp, vp, vp, vp, vp,
                                               vp, vp, vp, sz, vp]
    lib.moe_ffn_backward.argtypes = [P(MoeShape), P(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, P(MoeSaved), vp, vp, P(MoeGrads), vp, sz, vp]
    lib.moe_balance_counts.argtypes = [P(MoeShape), vp, vp, vp, ctypes.c_float, vp]
    lib.moe_score_f32.argtypes = [i32, vp, vp, i64, vp]
    lib.moe_bandwidth_probe.argtypes = [i32, vp, vp, i64, i32, vp]
    lib.moe_profile_begin.argtypes = [i32]
    lib.moe_profile_end.argtypes = [P(ctypes.c_float), i32, P(ctypes.c_int)]
    lib.moe_workspace_bytes.argtypes = [P(MoeShape), i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_status_str.argtypes = [i32]
    lib.moe_status_str.restype = ctypes.c_char_p
    for f in ("moe_route", "moe_dispatch", "moe_route_dispatch", "moe_ffn_forward", "moe_layer_forward",
              "moe_ffn_forward_noalloc", "moe_ffn_forward_partial",
              "moe_combine",
              "moe_parallel_block_forward", "moe_ffn_backward", "moe_aux_loss",
              "moe_balance_counts", "moe_score_f32", "moe_bandwidth_probe", "moe_profile_begin",
              "moe_profile_end"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def make_shape(T, H, E, k, I, Is=0, score=SCORE_SOFTMAX, renorm=True, shared_gated=False,
               dtype=DTYPE_BF16) -> MoeShape:
    return MoeShape(int(T), int(H), int(E), int(k), int(I), int(Is), int(score), int(bool(renorm)),
                    int(bool(shared_gated)), int(dtype))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def workspace_bytes(shape: MoeShape, op: int) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(shape), op))


def _nbytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def moe_route(shape: MoeShape, x, w_router, w_shared_gate, sel_bias, logits, weights, ids, gate,
              flags: int = 0, stream=None, score_sums=None, ws=None) -> None:
    _check("moe_route", load().moe_route(
        ctypes.byref(shape), _p(x), _p(w_router), _p(w_shared_gate), _p(sel_bias), _p(logits),
        _p(weights), _p(ids), _p(gate), _p(score_sums), _p(ws), _nbytes(ws), int(flags), _stream(stream)))


def moe_aux_loss(shape: MoeShape, score_sums, counts, alpha: float, loss, coef, stream=None) -> None:
    _check("moe_aux_loss", load().moe_aux_loss(
        ctypes.byref(shape), _p(score_sums), _p(counts), ctypes.c_float(alpha), _p(loss), _p(coef),
        _stream(stream)))


def moe_dispatch(shape: MoeShape, ids, x, counts, offsets, perm, pos, x_sorted, ws, stream=None) -> None:
    _check("moe_dispatch", load().moe_dispatch(
        ctypes.byref(shape), _p(ids), _p(x), _p(counts), _p(offsets), _p(perm), _p(pos),
        _p(x_sorted), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_dispatch(shape: MoeShape, x, w_router, w_shared_gate, sel_bias, logits, weights, ids, gate,
                       counts, offsets, perm, pos, ws, flags: int = 0, stream=None, score_sums=None) -> None:
    _check("moe_route_dispatch", load().moe_route_dispatch(
        ctypes.byref(shape), _p(x), _p(w_router), _p(w_shared_gate), _p(sel_bias), _p(logits), _p(weights),
        _p(ids), _p(gate), _p(score_sums), _p(counts), _p(offsets), _p(perm), _p(pos), _p(ws), _nbytes(ws),
        int(flags), _stream(stream)))


def weights_struct(w_gate_up, w_down, ws_gate_up=None, ws_down=None, w_shared_gate=None) -> MoeWeights:
    return MoeWeights(_p(w_gate_up), _p(w_down), _p(ws_gate_up), _p(ws_down), _p(w_shared_gate))


def saved_struct(gu=None, h=None, y=None, s_gu=None, s_h=None, s_y=None) -> MoeSaved:
    return MoeSaved(_p(gu), _p(h), _p(y), _p(s_gu), _p(s_h), _p(s_y))


def grads_struct(dx, dw_router, dw_gate_up, dw_down, dws_gate_up=None, dws_down=None,
                 dw_shared_gate=None, dlogits=None) -> MoeGrads:
    return MoeGrads(_p(dx), _p(dw_router), _p(dw_gate_up), _p(dw_down), _p(dws_gate_up),
                    _p(dws_down), _p(dw_shared_gate), _p(dlogits))


def moe_ffn_forward(shape: MoeShape, weights: MoeWeights, x, x_sorted, offsets, perm, pos, routing_weights,
                    gate, out, saved: Optional[MoeSaved], ws, stream=None) -> None:
    _check("moe_ffn_forward", load().moe_ffn_forward(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), _p(x_sorted), _p(offsets), _p(perm), _p(pos),
        _p(routing_weights), _p(gate), _p(out), None if saved is None else ctypes.byref(saved),
        _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_forward(shape: MoeShape, weights: MoeWeights, x, w_router, w_shared_gate, sel_bias, routing_weights,
                      ids, gate, counts, offsets, perm, pos, out, ws, stream=None) -> None:
    _check("moe_layer_forward", load().moe_layer_forward(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), _p(w_router), _p(w_shared_gate), _p(sel_bias),
        _p(routing_weights), _p(ids), _p(gate), _p(counts), _p(offsets), _p(perm), _p(pos), _p(out), _p(ws),
        _nbytes(ws), _stream(stream)))


def moe_ffn_forward_noalloc(shape: MoeShape, weights: MoeWeights, x, x_sorted, offsets, perm, pos, routing_weights,
                            gate, out, stream=None) -> None:
    _check("moe_ffn_forward_noalloc", load().moe_ffn_forward_noalloc(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), _p(x_sorted), _p(offsets), _p(perm), _p(pos),
        _p(routing_weights), _p(gate), _p(out), _stream(stream)))


def moe_ffn_forward_partial(shape: MoeShape, weights: MoeWeights, x, x_sorted, offsets, perm, y_part, s_part,
                            saved: Optional[MoeSaved], ws, stream=None) -> None:
    _check("moe_ffn_forward_partial", load().moe_ffn_forward_partial(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), _p(x_sorted), _p(offsets), _p(perm), _p(y_part),
        _p(s_part), None if saved is None else ctypes.byref(saved), _p(ws), _nbytes(ws), _stream(stream)))


def moe_combine(shape: MoeShape, y, pos, routing_weights, gate, s_y, out, stream=None) -> None:
    _check("moe_combine", load().moe_combine(
        ctypes.byref(shape), _p(y), _p(pos), _p(routing_weights), _p(gate), _p(s_y), _p(out), _stream(stream)))


def block_norms(g_pre_moe, g_post_dense, g_post_moe, g_post, eps: float, layer_scalar: float) -> MoeBlockNorms:
    return MoeBlockNorms(_p(g_pre_moe), _p(g_post_dense), _p(g_post_moe), _p(g_post), float(eps),
                         float(layer_scalar))


def moe_parallel_block_forward(shape: MoeShape, weights: MoeWeights, norms: MoeBlockNorms, residual, x_dense,
                               offsets, perm, pos, routing_weights, out, ws, stream=None) -> None:
    _check("moe_parallel_block_forward", load().moe_parallel_block_forward(
        ctypes.byref(shape), ctypes.byref(weights), ctypes.byref(norms), _p(residual), _p(x_dense), _p(offsets),
        _p(perm), _p(pos), _p(routing_weights), _p(out), _p(ws), _nbytes(ws), _stream(stream)))


def moe_ffn_backward(shape: MoeShape, weights: MoeWeights, x, w_router, logits, ids, routing_weights, gate,
                     offsets, perm, pos, x_sorted, saved: MoeSaved, dout, grads: MoeGrads, ws,
                     stream=None, aux_coef=None) -> None:
    _check("moe_ffn_backward", load().moe_ffn_backward(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), _p(w_router), _p(logits), _p(ids),
        _p(routing_weights), _p(gate), _p(offsets), _p(perm), _p(pos), _p(x_sorted), ctypes.byref(saved),
        _p(dout), _p(aux_coef), ctypes.byref(grads), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_balance_counts(shape: MoeShape, ids, counts, bias, rate: float, stream=None) -> None:
    _check("moe_balance_counts", load().moe_balance_counts(
        ctypes.byref(shape), _p(ids), _p(counts), _p(bias), ctypes.c_float(rate), _stream(stream)))


def moe_score_f32(score: int, logits, out, stream=None) -> None:
    _check("moe_score_f32", load().moe_score_f32(int(score), _p(logits), _p(out), int(logits.numel()),
                                                 _stream(stream)))


def moe_bandwidth_probe(kind: int, src, dst, nbytes: int, wgs: int = 0, stream=None) -> None:
    """kind 0: read src (dst gets one word per thread), 1: write dst, 2: copy src -> dst."""
    _check("moe_bandwidth_probe", load().moe_bandwidth_probe(int(kind), _p(src) if src is not None else None,
                                                             _p(dst), int(nbytes), int(wgs), _stream(stream)))


def moe_profile_begin(max_calls: int) -> None:
    _check("moe_profile_begin", load().moe_profile_begin(int(max_calls)))


def moe_profile_end():
    """Returns ({stage name: summed ms}, n_forward_calls, n_backward_calls)."""
    ms = (ctypes.c_float * N_STAGES)()
    calls = (ctypes.c_int * 2)()
    _check("moe_profile_end", load().moe_profile_end(ms, N_STAGES, calls))
    return {n: float(ms[i]) for i, n in enumerate(STAGE_NAMES)}, int(calls[0]), int(calls[1])
