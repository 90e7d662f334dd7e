"""torch-facing binding of the C ABI: allocation, checks and argument
marshalling only.  Every step of routing, forward and backward runs in the
HIP kernels of ``libmoe_lora.so``; nothing here computes."""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass
from typing import NamedTuple, Optional

import torch

from . import _lib


@dataclass(frozen=True)
class Dims:
    """Layer shape (see moe_dims in include/moe_lora.h)."""

    T: int
    d: int
    n: int
    E: int
    k: int
    r: int
    n_shared: int = 0
    lora_scale: float = 1.0
    dtype: int = _lib.MOE_BF16  # element type of x, y, dy, dx and the weights

    @property
    def elem(self) -> torch.dtype:
        """torch dtype of the 16-bit tensors (activations and weights)."""
        if self.dtype == _lib.MOE_BF16:
            return torch.bfloat16
        if self.dtype == _lib.MOE_F16:
            return torch.float16
        raise ValueError(f"unknown element type {self.dtype}")

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def P_tot(self) -> int:
        return self.T * self.k + self.n_shared * self.T

    @property
    def E_tot(self) -> int:
        return self.E + self.n_shared

    def c(self) -> _lib.MoeDims:
        return _lib.MoeDims(self.T, self.d, self.n, self.E, self.k, self.r, self.n_shared,
                            float(self.lora_scale), int(self.dtype))


class Routing(NamedTuple):
    topk_ids: torch.Tensor     # int32 [T, k]
    topk_w: torch.Tensor       # fp32  [T, k]
    counts: torch.Tensor       # int32 [E]
    offsets: torch.Tensor      # int32 [E+1]
    sorted_pair: torch.Tensor  # int32 [P]
    pair_pos: torch.Tensor     # int32 [P]
    row_token: torch.Tensor    # int32 [P_tot] token of each sorted row
    row_weight: torch.Tensor   # fp32  [P_tot] routing weight of each sorted row


class Weights(NamedTuple):
    """Frozen base weights and LoRA factors, all of the layer's element type."""
    w_gate_up: torch.Tensor  # [E_tot, 2n, d]
    w_down: torch.Tensor     # [E_tot, d, n]
    a_gate_up: torch.Tensor  # [E_tot, d, r]
    b_gate_up: torch.Tensor  # [E_tot, r, 2n]
    a_down: torch.Tensor     # [E_tot, n, r]
    b_down: torch.Tensor     # [E_tot, r, d]


class Grads(NamedTuple):
    dx: torch.Tensor          # element type [T, d]
    da_gate_up: torch.Tensor  # fp32 [E_tot, d, r]
    db_gate_up: torch.Tensor  # fp32 [E_tot, r, 2n]
    da_down: torch.Tensor     # fp32 [E_tot, n, r]
    db_down: torch.Tensor     # fp32 [E_tot, r, d]


class RouterGrads(NamedTuple):
    """Gradients that reach the router, for models that train it."""
    d_topk_w: torch.Tensor    # fp32 [T, k]
    d_logits: torch.Tensor    # fp32 [T, E]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, shape, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@contextlib.contextmanager
def _on(stream):
    """Allocations and the library call of one wrapper, on ``stream`` (None =
    the current stream).  A stream other than the current one first waits for
    the current stream, where the inputs were produced; tensors allocated
    inside belong to that stream's pool, so the caching allocator does not hand
    their memory to other work while the enqueued kernels may still use it.
    Outputs allocated here are ready on ``stream``; a caller that reads them on
    another stream orders it after ``stream`` itself."""
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        yield cur.cuda_stream
        return
    stream.wait_stream(cur)
    with torch.cuda.stream(stream):
        yield stream.cuda_stream


def route_workspace_bytes(dims: Dims) -> int:
    dc = dims.c()
    return _lib.load().moe_route_workspace_bytes(ctypes.byref(dc))


def forward_saved_bytes(dims: Dims) -> int:
    dc = dims.c()
    return _lib.load().moe_forward_saved_bytes(ctypes.byref(dc))


def workspace_bytes(dims: Dims) -> int:
    dc = dims.c()
    return _lib.load().moe_workspace_bytes(ctypes.byref(dc))


def _bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def empty_routing(dims: Dims, device) -> Routing:
    i32 = torch.int32
    return Routing(torch.empty(dims.T, dims.k, dtype=i32, device=device),
                   torch.empty(dims.T, dims.k, dtype=torch.float32, device=device),
                   torch.empty(dims.E, dtype=i32, device=device),
                   torch.empty(dims.E + 1, dtype=i32, device=device),
                   torch.empty(dims.P, dtype=i32, device=device),
                   torch.empty(dims.P, dtype=i32, device=device),
                   torch.empty(dims.P_tot, dtype=i32, device=device),
                   torch.empty(dims.P_tot, dtype=torch.float32, device=device))


def _c_routing(rt: Routing) -> _lib.MoeRouting:
    return _lib.MoeRouting(*[t.data_ptr() for t in rt])


def _c_weights(w: Weights) -> _lib.MoeWeights:
    return _lib.MoeWeights(*[t.data_ptr() for t in w])


def _check_routing(rt: Routing, dims: Dims) -> None:
    i32 = torch.int32
    _check(rt.topk_ids, (dims.T, dims.k), i32, "topk_ids")
    _check(rt.topk_w, (dims.T, dims.k), torch.float32, "topk_w")
    _check(rt.counts, (dims.E,), i32, "counts")
    _check(rt.offsets, (dims.E + 1,), i32, "offsets")
    _check(rt.sorted_pair, (dims.P,), i32, "sorted_pair")
    _check(rt.pair_pos, (dims.P,), i32, "pair_pos")
    _check(rt.row_token, (dims.P_tot,), i32, "row_token")
    _check(rt.row_weight, (dims.P_tot,), torch.float32, "row_weight")


def _check_weights(w: Weights, dims: Dims) -> None:
    bf, Et, d, n, r = dims.elem, dims.E_tot, dims.d, dims.n, dims.r
    _check(w.w_gate_up, (Et, 2 * n, d), bf, "w_gate_up")
    _check(w.w_down, (Et, d, n), bf, "w_down")
    _check(w.a_gate_up, (Et, d, r), bf, "a_gate_up")
    _check(w.b_gate_up, (Et, r, 2 * n), bf, "b_gate_up")
    _check(w.a_down, (Et, n, r), bf, "a_down")
    _check(w.b_down, (Et, r, d), bf, "b_down")


def route(logits: torch.Tensor, dims: Dims, out: Optional[Routing] = None,
          ws: Optional[torch.Tensor] = None, stream=None) -> Routing:
    """moe_route: top-k softmax routing and the one-pass grouping."""
    lib = _lib.load()
    _check(logits, (dims.T, dims.E), torch.float32, "logits")
    with _on(stream) as s:
        out = out if out is not None else empty_routing(dims, logits.device)
        _check_routing(out, dims)
        if ws is None:
            ws = _bytes(route_workspace_bytes(dims), logits.device)
        dc, rc = dims.c(), _c_routing(out)
        _lib.check(lib.moe_route(ctypes.byref(dc), logits.data_ptr(), ctypes.byref(rc), ws.data_ptr(),
                                 ws.numel(), s), "moe_route")
    return out


def route_noalloc(logits: torch.Tensor, dims: Dims, out: Routing, stream=None) -> Routing:
    """moe_route_noalloc: routing into caller-owned buffers with the library's
    own per-GPU scratch (no workspace; nothing is allocated).  Calls that
    overlap on one GPU race."""
    lib = _lib.load()
    _check(logits, (dims.T, dims.E), torch.float32, "logits")
    _check_routing(out, dims)
    dc, rc = dims.c(), _c_routing(out)
    with _on(stream) as s:
        _lib.check(lib.moe_route_noalloc(ctypes.byref(dc), logits.data_ptr(), ctypes.byref(rc), s),
                   "moe_route_noalloc")
    return out


def forward(x: torch.Tensor, routing: Routing, weights: Weights, dims: Dims,
            y: Optional[torch.Tensor] = None, saved: Optional[torch.Tensor] = None,
            ws: Optional[torch.Tensor] = None, stream=None):
    """moe_lora_forward.  Returns (y, saved); keep `saved` for backward."""
    lib = _lib.load()
    _check(x, (dims.T, dims.d), dims.elem, "x")
    _check_routing(routing, dims)
    _check_weights(weights, dims)
    with _on(stream) as s:
        y = y if y is not None else torch.empty_like(x)
        _check(y, (dims.T, dims.d), dims.elem, "y")
        if saved is None:
            saved = _bytes(forward_saved_bytes(dims), x.device)
        if ws is None:
            ws = _bytes(workspace_bytes(dims), x.device)
        dc, rc, wc = dims.c(), _c_routing(routing), _c_weights(weights)
        _lib.check(lib.moe_lora_forward(ctypes.byref(dc), x.data_ptr(), ctypes.byref(rc),
                                        ctypes.byref(wc), y.data_ptr(), saved.data_ptr(),
                                        saved.numel(), ws.data_ptr(), ws.numel(), s),
                   "moe_lora_forward")
    return y, saved


def empty_grads(dims: Dims, device) -> Grads:
    f32, Et, d, n, r = torch.float32, dims.E_tot, dims.d, dims.n, dims.r
    return Grads(torch.empty(dims.T, d, dtype=dims.elem, device=device),
                 torch.empty(Et, d, r, dtype=f32, device=device),
                 torch.empty(Et, r, 2 * n, dtype=f32, device=device),
                 torch.empty(Et, n, r, dtype=f32, device=device),
                 torch.empty(Et, r, d, dtype=f32, device=device))


def empty_router_grads(dims: Dims, device) -> RouterGrads:
    return RouterGrads(torch.empty(dims.T, dims.k, dtype=torch.float32, device=device),
                       torch.empty(dims.T, dims.E, dtype=torch.float32, device=device))


def backward(dy: torch.Tensor, x: torch.Tensor, routing: Routing, weights: Weights,
             saved: torch.Tensor, dims: Dims, out: Optional[Grads] = None,
             ws: Optional[torch.Tensor] = None, stream=None,
             router_out: Optional[RouterGrads] = None) -> Grads:
    """moe_lora_backward: dX and the LoRA-factor gradients; with ``router_out``
    also the routing-weight and logit gradients (written into it)."""
    lib = _lib.load()
    _check(dy, (dims.T, dims.d), dims.elem, "dy")
    _check(x, (dims.T, dims.d), dims.elem, "x")
    _check_routing(routing, dims)
    _check_weights(weights, dims)
    Et, d, n, r = dims.E_tot, dims.d, dims.n, dims.r
    dtw = dlg = None
    if router_out is not None:
        _check(router_out.d_topk_w, (dims.T, dims.k), torch.float32, "d_topk_w")
        _check(router_out.d_logits, (dims.T, dims.E), torch.float32, "d_logits")
        dtw, dlg = router_out.d_topk_w.data_ptr(), router_out.d_logits.data_ptr()
    with _on(stream) as s:
        out = out if out is not None else empty_grads(dims, dy.device)
        _check(out.dx, (dims.T, d), dims.elem, "dx")
        _check(out.da_gate_up, (Et, d, r), torch.float32, "da_gate_up")
        _check(out.db_gate_up, (Et, r, 2 * n), torch.float32, "db_gate_up")
        _check(out.da_down, (Et, n, r), torch.float32, "da_down")
        _check(out.db_down, (Et, r, d), torch.float32, "db_down")
        if ws is None:
            ws = _bytes(workspace_bytes(dims), dy.device)
        dc, rc, wc = dims.c(), _c_routing(routing), _c_weights(weights)
        _lib.check(lib.moe_lora_backward(ctypes.byref(dc), dy.data_ptr(), x.data_ptr(),
                                         ctypes.byref(rc), ctypes.byref(wc), saved.data_ptr(),
                                         saved.numel(), out.dx.data_ptr(), out.da_gate_up.data_ptr(),
                                         out.db_gate_up.data_ptr(), out.da_down.data_ptr(),
                                         out.db_down.data_ptr(), dtw, dlg, ws.data_ptr(), ws.numel(),
                                         s),
                   "moe_lora_backward")
    return out


class MergedWeights(NamedTuple):
    """Base weights with the LoRA delta merged in (the path split LoRA avoids)."""
    w_gate_up: torch.Tensor  # [E_tot, 2n, d]
    w_down: torch.Tensor     # [E_tot, d, n]


def merge_lora(weights: Weights, dims: Dims, out: Optional[MergedWeights] = None,
               stream=None) -> MergedWeights:
    """moe_merge_lora: W + s (A B)^T of every expert, both modules."""
    lib = _lib.load()
    _check_weights(weights, dims)
    with _on(stream) as s:
        if out is None:
            out = MergedWeights(torch.empty_like(weights.w_gate_up), torch.empty_like(weights.w_down))
        _check(out.w_gate_up, tuple(weights.w_gate_up.shape), dims.elem, "w_gate_up_merged")
        _check(out.w_down, tuple(weights.w_down.shape), dims.elem, "w_down_merged")
        dc, wc = dims.c(), _c_weights(weights)
        _lib.check(lib.moe_merge_lora(ctypes.byref(dc), ctypes.byref(wc), out.w_gate_up.data_ptr(),
                                      out.w_down.data_ptr(), s), "moe_merge_lora")
    return out


def forward_merged(x: torch.Tensor, routing: Routing, merged: MergedWeights, dims: Dims,
                   y: Optional[torch.Tensor] = None, saved: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_forward_merged: the forward on merged weights, low-rank pass off."""
    lib = _lib.load()
    Et, d, n = dims.E_tot, dims.d, dims.n
    _check(x, (dims.T, d), dims.elem, "x")
    _check_routing(routing, dims)
    _check(merged.w_gate_up, (Et, 2 * n, d), dims.elem, "w_gate_up_merged")
    _check(merged.w_down, (Et, d, n), dims.elem, "w_down_merged")
    with _on(stream) as s:
        y = y if y is not None else torch.empty_like(x)
        _check(y, (dims.T, d), dims.elem, "y")
        if saved is None:
            saved = _bytes(forward_saved_bytes(dims), x.device)
        if ws is None:
            ws = _bytes(workspace_bytes(dims), x.device)
        dc, rc = dims.c(), _c_routing(routing)
        _lib.check(lib.moe_forward_merged(ctypes.byref(dc), x.data_ptr(), ctypes.byref(rc),
                                          merged.w_gate_up.data_ptr(), merged.w_down.data_ptr(),
                                          y.data_ptr(), saved.data_ptr(), saved.numel(),
                                          ws.data_ptr(), ws.numel(), s), "moe_forward_merged")
    return y


ENGINE_GATE_UP, ENGINE_DOWN, ENGINE_DH, ENGINE_DX, ENGINE_RANK = 1, 2, 4, 8, 16
ENGINE_ALL = 31          # every product streamed, default tiles (MOE_ENGINE_DEFAULT)
PRODUCTS = ("gate_up", "down", "dh", "dx")
SPLITK_1024, SPLITK_4096 = 1 << 13, 2 << 13


def TILE256(p: int) -> int:
    """Engine bit: 256-row tiles (else 320) for product p (0 gate_up, 1 down, 2 dh, 3 dx)."""
    return 1 << (5 + p)


def STAGE32(p: int) -> int:
    """Engine bit: 32-k ring stages (else 64-k) for product p."""
    return 1 << (9 + p)


def describe_engines(bits: int) -> dict:
    """Readable form of an engine/tile word."""
    out = {}
    for p, name in enumerate(PRODUCTS):
        if bits & (1 << p):
            out[name] = (f"streamed {256 if bits & TILE256(p) else 320}x256 "
                         f"{32 if bits & STAGE32(p) else 64}-k")
        else:
            out[name] = "register-path"
    f = (bits >> 13) & 3
    out["rank_r"] = ("streamed" if bits & ENGINE_RANK else "register-path") + \
        f", split-K {({0: 2048, 1: 1024, 2: 4096}).get(f, '?')} rows"
    return out


def set_engines(dims: Dims, engines: int) -> None:
    """Record the engines for this layer shape (bit set = streamed kernels)."""
    lib = _lib.load()
    dc = dims.c()
    _lib.check(lib.moe_set_engines(ctypes.byref(dc), int(engines)), "moe_set_engines")


def get_engines(dims: Dims) -> int:
    lib = _lib.load()
    dc = dims.c()
    return int(lib.moe_get_engines(ctypes.byref(dc)))


def autotune(dims: Dims, logits: torch.Tensor, x: torch.Tensor, dy: torch.Tensor,
             weights: Weights, stream=None) -> int:
    """One-time per-shape engine autotune (waits for the GPU); returns and
    records the chosen engine bits."""
    lib = _lib.load()
    _check(logits, (dims.T, dims.E), torch.float32, "logits")
    _check(x, (dims.T, dims.d), dims.elem, "x")
    _check(dy, (dims.T, dims.d), dims.elem, "dy")
    _check_weights(weights, dims)
    dc, wc = dims.c(), _c_weights(weights)
    out = ctypes.c_uint(0)
    with _on(stream) as s:
        scratch = _bytes(int(lib.moe_autotune_scratch_bytes(ctypes.byref(dc))), x.device)
        _lib.check(lib.moe_autotune(ctypes.byref(dc), logits.data_ptr(), x.data_ptr(), dy.data_ptr(),
                                    ctypes.byref(wc), scratch.data_ptr(), scratch.numel(),
                                    s, ctypes.byref(out)), "moe_autotune")
    return int(out.value)


class MoELoRALayer:
    """One layer with every buffer allocated up front, so that route / forward /
    backward allocate nothing per call (the benchmark's steady state)."""

    def __init__(self, dims: Dims, weights: Weights, device="cuda"):
        _check_weights(weights, dims)
        self.dims, self.weights = dims, weights
        self.routing = empty_routing(dims, device)
        self.route_ws = _bytes(route_workspace_bytes(dims), device)
        self.saved = _bytes(forward_saved_bytes(dims), device)
        self.ws = _bytes(workspace_bytes(dims), device)
        self.y = torch.empty(dims.T, dims.d, dtype=dims.elem, device=device)
        self.grads = empty_grads(dims, device)
        self.router_grads: Optional[RouterGrads] = None

    def route(self, logits, stream=None) -> Routing:
        return route(logits, self.dims, self.routing, self.route_ws, stream)

    def forward(self, x, stream=None) -> torch.Tensor:
        forward(x, self.routing, self.weights, self.dims, self.y, self.saved, self.ws, stream)
        return self.y

    def backward(self, dy, x, stream=None, router: bool = False) -> Grads:
        """dX and the LoRA gradients; with ``router`` also ``self.router_grads``."""
        if router and self.router_grads is None:
            self.router_grads = empty_router_grads(self.dims, self.y.device)
        return backward(dy, x, self.routing, self.weights, self.saved, self.dims, self.grads,
                        self.ws, stream, self.router_grads if router else None)
