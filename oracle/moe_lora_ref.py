"""Plain, slow CPU oracle for the MoE expert layer with split LoRA.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it; the only thing both sides
share is the seeded input generator in ``synth``.

Sources (two web pages; cited by title and section):

[ROUTE] Chinese-language article on three Unsloth x NVIDIA training
        optimisations (m.yhxrc.cn), section "Optimisation 3: MoE routing grouped
        once" -- the per-expert ``torch.where`` loop it replaces, and the
        replacement recipe: flatten the top-k assignments, stable-sort by expert
        id, one bincount for per-expert counts, offsets from the counts, slice
        the sorted list by offset; the routing logic itself is unchanged.
[MOE]   Unsloth documentation page "Fine-tune MoE models 12x faster with
        Unsloth" (faster-moe), sections
          "What is torch._grouped_mm?" -- experts stored as one parameter
              [E, 2*intermediate, hidden]; per expert ``linear`` then
              ``chunk(2, dim=-1)`` into gate and up;
          "Faster LoRA MoE training" -- split LoRA computes the base product and
              the low-rank product separately instead of merging the adapter
              into the weight; identical in exact arithmetic (associativity),
              so outputs, loss and gradients are unchanged; the router is not
              trained;
          "Implementation details" / "MoE LoRA changes things" -- LoRA on a
              weight of shape (m, n) adds A (m, r) and B (r, n); the split
              path computes (X A) B per routed (token, expert) pair.

Readings taken where the pages are silent (each is pinned or declared in the
tests):
  * top-k order: descending logit, equal logits -> lower expert id first;
  * routing weights: softmax over the k selected logits;
  * offsets: exclusive, length E+1, offsets[E] = T*k;
  * gate = rows [0, n) of the fused gate_up weight, up = rows [n, 2n)
    (contiguous halves, as ``chunk(2, dim=-1)`` splits them);
  * activation: SwiGLU, h = silu(gate) * up, silu(x) = x / (1 + exp(-x))
    (Shazeer, "GLU Variants Improve Transformer", 2020) -- the pages do not name
    the activation: parity unpinned by the pages, fixed by definition;
  * LoRA storage: A_gu [E,d,r], B_gu [E,r,2n], A_dn [E,n,r], B_dn [E,r,d]
    (the (m, r) / (r, n) shapes of the implementation-details section, with
    m = layer input, n = layer output); the delta of a weight stored
    [out, in] is s * (A B)^T;
  * LoRA scale s is an explicit argument (the pages set alpha = 2r in code but
    do not say how alpha is applied);
  * one shared expert, when present, is stacked as expert E with weight 1 for
    every token and is not routed;
  * the router is frozen in the layer's backward: it produces no gradient for
    logits or routing weights, none for the frozen base weights;
    ``router_grads`` gives the routing-weight and logit gradients separately,
    for a model whose router is trained (the selection is taken as locally
    constant, the shared expert's weight as the constant 1).

Arithmetic: float64 by default (float32 on request, used for timing); the
16-bit inputs (bf16, or IEEE fp16 for a layer whose element type is "f16")
are decoded exactly; no intermediate rounding.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Routing",
    "bf16_decode",
    "f16_decode",
    "decode",
    "topk_softmax",
    "route",
    "route_naive",
    "gather_rows",
    "silu",
    "expert_forward",
    "forward",
    "forward_naive",
    "forward_merged",
    "merged_weights",
    "forward_tokens",
    "backward",
    "backward_tokens",
    "lora_grads_expert",
    "router_grads",
    "router_grads_tokens",
]


def bf16_decode(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float values.

    Arrays that are already floating point are only cast, so the oracle can be
    driven with perturbed real-valued inputs (finite differences)."""
    a = np.asarray(bits)
    if a.dtype != np.uint16:
        return a.astype(dtype, copy=False)
    u = a.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype, copy=False)


def f16_decode(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """IEEE 754 binary16 bit patterns (uint16) -> exact float values.

    Written from the format's definition: sign bit, 5-bit exponent with bias
    15, 10-bit fraction; exponent 0 holds the subnormals (fraction * 2^-24),
    exponent 31 infinities and NaNs.  Floating-point arrays are only cast."""
    a = np.asarray(bits)
    if a.dtype != np.uint16:
        return a.astype(dtype, copy=False)
    u = a.astype(np.int64)
    sign = np.where(u >> 15, -1.0, 1.0)
    ex = (u >> 10) & 0x1F
    fr = (u & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + fr / 1024.0, ex - 15)
    sub = np.ldexp(fr, -24)
    special = np.where(fr == 0, np.inf, np.nan)
    v = np.where(ex == 0, sub, np.where(ex == 31, special, normal))
    return (sign * v).astype(dtype, copy=False)


_DECODERS = {"bf16": bf16_decode, "f16": f16_decode}


def decode(inp, name: str, dtype=np.float64) -> np.ndarray:
    """Exact values of the 16-bit input array ``name`` of ``inp``, read in the
    layer's element type (``inp.dims.element``; bf16 when absent)."""
    element = getattr(inp.dims, "element", "bf16")
    return _DECODERS[element](getattr(inp, name), dtype)


# ----------------------------------------------------------------------------
# Routing  [ROUTE]
# ----------------------------------------------------------------------------

def topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their routing weights.

    ids[t] lists the k experts with the largest logits, largest first; equal
    logits are ordered by ascending expert id.  w[t, j] is the softmax of the k
    selected logits, evaluated in float64 relative to the largest one and
    rounded to float32.

    Non-finite logits (outside what the pages consider): NaN ranks below every
    other value, -inf included, and NaNs tie with each other (lower id first),
    so every id is a valid expert.  The weights of a token whose selected
    logits are not all finite are whatever the softmax formula gives (NaN when
    a NaN or an infinite maximum enters).  numpy's sort places NaN keys last,
    which is exactly this order for the negated logits.
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    eid = np.broadcast_to(np.arange(E, dtype=np.int64), L.shape)
    # lexsort: last key is primary (descending logit), then ascending id.
    order = np.lexsort((eid, -L), axis=-1)
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


@dataclass
class Routing:
    """Grouping of the T*k (token, slot) pairs by expert.

    counts[e]      pairs routed to expert e;
    offsets[e]     first sorted position of expert e (exclusive prefix sum,
                   length E+1, offsets[E] = T*k);
    sorted_pair[p] flat pair index t*k + j stored at sorted position p;
    pair_pos[i]    sorted position of flat pair i (inverse permutation).
    """

    counts: np.ndarray
    offsets: np.ndarray
    sorted_pair: np.ndarray
    pair_pos: np.ndarray


def route(topk_ids: np.ndarray, E: int) -> Routing:
    """The pages' one-pass grouping, step by step [ROUTE].

    1. flatten all assignments (flat index i = t*k + j);
    2. stable sort by expert id;
    3. one bincount gives the per-expert counts;
    4. offsets from the counts;
    5. expert e's pairs are the sorted list sliced at [offsets[e], offsets[e+1]).
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    sorted_pair = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(flat.size)
    return Routing(counts.astype(np.int32), offsets.astype(np.int32),
                   sorted_pair.astype(np.int32), pair_pos.astype(np.int32))


def gather_rows(R: Routing, topk_w: np.ndarray, T: int, k: int, n_shared: int = 0):
    """The gather step of the recipe [ROUTE]: the token and routing weight of
    every sorted row.  Row p < T*k holds pair sorted_pair[p] = t*k + j, i.e.
    token t with weight topk_w[t, j]; with a shared expert, rows T*k + t follow,
    token t with weight 1."""
    sp = R.sorted_pair.astype(np.int64)
    tok = sp // k
    wgt = np.asarray(topk_w, dtype=np.float32).reshape(-1)[sp]
    if n_shared:
        tok = np.concatenate([tok, np.arange(T)])
        wgt = np.concatenate([wgt, np.ones(T, np.float32)])
    return tok.astype(np.int32), wgt.astype(np.float32)


def route_naive(topk_ids: np.ndarray, E: int):
    """The per-expert loop the recipe replaces [ROUTE]: for every expert, find
    the (token, slot) entries equal to it.  Returns, per expert, the token
    indices and slots in the order the search yields them (ascending token)."""
    ids = np.asarray(topk_ids)
    out = []
    for e in range(E):
        tok, slot = np.nonzero(ids == e)
        out.append((tok, slot))
    return out


# ----------------------------------------------------------------------------
# Expert MLP with split LoRA  [MOE]
# ----------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _params(inp, dtype):
    return {name: decode(inp, name, dtype)
            for name in ("w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn")}


def expert_forward(xe, W, e, n, s):
    """Forward of expert e on the rows ``xe`` (shape [c, d]).

    G = X W_gu^T + s (X A_gu) B_gu; gate/up = the two halves of G's columns;
    H = silu(gate) * up; O = H W_dn^T + s (H A_dn) B_dn.
    Returns (G, H, O, XA, HA).
    """
    xa = xe @ W["a_gu"][e]
    g = xe @ W["w_gu"][e].T + s * (xa @ W["b_gu"][e])
    h = silu(g[:, :n]) * g[:, n:]
    ha = h @ W["a_dn"][e]
    o = h @ W["w_dn"][e].T + s * (ha @ W["b_dn"][e])
    return g, h, o, xa, ha


def _pairs_of_tokens(tokens, k):
    tokens = np.asarray(tokens, dtype=np.int64)
    return (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)


def forward(inp, topk_ids, topk_w, dims, dtype=np.float64, keep=False):
    """Whole-layer forward, grouped the pages' way (sorted pairs per expert).

    Y[t] = sum_j w[t, j] * O(t, expert j)  (+ the shared expert's O(t), weight 1),
    summed in slot order.  With ``keep`` also returns per-pair intermediates
    indexed by flat pair (shared rows after the routed ones).
    """
    T, d, n, k, E = dims.T, dims.d, dims.n, dims.k, dims.E
    s = dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    R = route(topk_ids, E)
    P = T * k
    P_tot = dims.P_tot
    o_pair = np.zeros((P_tot, d), dtype)
    saved = {}
    if keep:
        saved = {"g": np.zeros((P_tot, 2 * n), dtype), "h": np.zeros((P_tot, n), dtype),
                 "xa": np.zeros((P_tot, dims.r), dtype), "ha": np.zeros((P_tot, dims.r), dtype)}
    for e in range(dims.E_tot):
        if e < E:
            pairs = R.sorted_pair[R.offsets[e]:R.offsets[e + 1]].astype(np.int64)
            tok = pairs // k
        else:
            tok = np.arange(T)
            pairs = P + tok
        if pairs.size == 0:
            continue
        g, h, o, xa, ha = expert_forward(X[tok], W, e, n, s)
        o_pair[pairs] = o
        if keep:
            saved["g"][pairs], saved["h"][pairs] = g, h
            saved["xa"][pairs], saved["ha"][pairs] = xa, ha
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    y = np.zeros((T, d), dtype)
    for j in range(k):
        y += w[:, j:j + 1] * o_pair[np.arange(T) * k + j]
    if dims.n_shared:
        y += o_pair[P:P + T]
    out = {"y": y, "o_pair": o_pair, "routing": R}
    out.update(saved)
    return out


def forward_naive(inp, topk_ids, topk_w, dims, dtype=np.float64):
    """Forward written as the per-expert search loop the pages start from:
    every expert finds its (token, slot) entries, runs its MLP on those tokens
    and adds the weighted result into Y."""
    T, d, n, E = dims.T, dims.d, dims.n, dims.E
    s = dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    y = np.zeros((T, d), dtype)
    for e, (tok, slot) in enumerate(route_naive(topk_ids, E)):
        if tok.size == 0:
            continue
        o = expert_forward(X[tok], W, e, n, s)[2]
        np.add.at(y, tok, w[tok, slot][:, None] * o)
    for e in range(E, dims.E_tot):
        y += expert_forward(X, W, e, n, s)[2]
    return y


def merged_weights(inp, dims, dtype=np.float64):
    """The merged weights PEFT forms [MOE]: per expert e,
    W'_gu[e] = W_gu[e] + s (A_gu[e] B_gu[e])^T  ([2n, d]) and
    W'_dn[e] = W_dn[e] + s (A_dn[e] B_dn[e])^T  ([d, n])."""
    s = dims.lora_scale
    W = _params(inp, dtype)
    wgu = W["w_gu"] + s * np.transpose(W["a_gu"] @ W["b_gu"], (0, 2, 1))
    wdn = W["w_dn"] + s * np.transpose(W["a_dn"] @ W["b_dn"], (0, 2, 1))
    return wgu, wdn


def forward_merged(inp, topk_ids, topk_w, dims, dtype=np.float64):
    """Forward on merged weights W' = W + s (A B)^T -- the path split LoRA
    avoids.  Identical to ``forward`` in exact arithmetic [MOE]."""
    T, d, n, E = dims.T, dims.d, dims.n, dims.E
    X = decode(inp, "x", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    WGU, WDN = merged_weights(inp, dims, dtype)
    y = np.zeros((T, d), dtype)
    for e, (tok, slot) in enumerate(route_naive(topk_ids, dims.E_tot)):
        if e >= E:
            tok, slot = np.arange(T), None
        if tok.size == 0:
            continue
        wgu, wdn = WGU[e], WDN[e]
        g = X[tok] @ wgu.T
        h = silu(g[:, :n]) * g[:, n:]
        o = h @ wdn.T
        scale = 1.0 if slot is None else w[tok, slot][:, None]
        np.add.at(y, tok, scale * o)
    return y


def forward_tokens(inp, topk_ids, topk_w, dims, tokens, dtype=np.float64):
    """Y rows for the listed tokens only (each from its own k pairs)."""
    n, k, s = dims.n, dims.k, dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    ids = np.asarray(topk_ids)
    out = np.zeros((len(tokens), dims.d), dtype)
    for i, t in enumerate(tokens):
        xt = X[t:t + 1]
        for j in range(k):
            out[i] += w[t, j] * expert_forward(xt, W, int(ids[t, j]), n, s)[2][0]
        for e in range(dims.E, dims.E_tot):
            out[i] += expert_forward(xt, W, e, n, s)[2][0]
    return out


# ----------------------------------------------------------------------------
# Backward: dX, dA, dB (base weights and router frozen)  [MOE]
# ----------------------------------------------------------------------------

def _expert_backward(xe, dO, W, e, n, s):
    """Backward of expert e on rows xe with upstream dO = w * dY[token].

    Returns (dX_rows, dA_gu, dB_gu, dA_dn, dB_dn) for this expert's rows:
      Q_dn = dO B_dn^T;  dH = dO W_dn + s Q_dn A_dn^T;
      dB_dn = s (H A_dn)^T dO;  dA_dn = s H^T Q_dn;
      dgate = dH * up * silu'(gate),  dup = dH * silu(gate),
      silu'(x) = sig(x) (1 + x (1 - sig(x)));
      Q_gu = dG B_gu^T;  dX = dG W_gu + s Q_gu A_gu^T;
      dB_gu = s (X A_gu)^T dG;  dA_gu = s X^T Q_gu.
    """
    g, h, _, xa, ha = expert_forward(xe, W, e, n, s)
    q_dn = dO @ W["b_dn"][e].T
    dh = dO @ W["w_dn"][e] + s * (q_dn @ W["a_dn"][e].T)
    db_dn = s * (ha.T @ dO)
    da_dn = s * (h.T @ q_dn)
    gate, up = g[:, :n], g[:, n:]
    sg = 1.0 / (1.0 + np.exp(-gate))
    dgate = dh * up * (sg * (1.0 + gate * (1.0 - sg)))
    dup = dh * (gate * sg)
    dg = np.concatenate([dgate, dup], axis=1)
    q_gu = dg @ W["b_gu"][e].T
    dx = dg @ W["w_gu"][e] + s * (q_gu @ W["a_gu"][e].T)
    db_gu = s * (xa.T @ dg)
    da_gu = s * (xe.T @ q_gu)
    return dx, da_gu, db_gu, da_dn, db_dn


def backward(inp, topk_ids, topk_w, dims, dtype=np.float64):
    """Whole-layer backward given dY (``inp.dy``).

    dX[t] = sum_j dX_pair(t, j) (+ shared), summed in slot order; the routing
    weight enters through dO = w * dY.  LoRA gradients are exactly zero for an
    expert that receives no rows.
    """
    T, d, n, r, k, E = dims.T, dims.d, dims.n, dims.r, dims.k, dims.E
    s = dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    dY = decode(inp, "dy", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype).reshape(-1)
    R = route(topk_ids, E)
    P = T * k
    Et = dims.E_tot
    dx_pair = np.zeros((dims.P_tot, d), dtype)
    grads = {"da_gu": np.zeros((Et, d, r), dtype), "db_gu": np.zeros((Et, r, 2 * n), dtype),
             "da_dn": np.zeros((Et, n, r), dtype), "db_dn": np.zeros((Et, r, d), dtype)}
    for e in range(Et):
        if e < E:
            pairs = R.sorted_pair[R.offsets[e]:R.offsets[e + 1]].astype(np.int64)
            tok = pairs // k
            wt = w[pairs][:, None]
        else:
            tok = np.arange(T)
            pairs = P + tok
            wt = 1.0
        if pairs.size == 0:
            continue
        dx, da_gu, db_gu, da_dn, db_dn = _expert_backward(X[tok], wt * dY[tok], W, e, n, s)
        dx_pair[pairs] = dx
        grads["da_gu"][e], grads["db_gu"][e] = da_gu, db_gu
        grads["da_dn"][e], grads["db_dn"][e] = da_dn, db_dn
    dxo = np.zeros((T, d), dtype)
    for j in range(k):
        dxo += dx_pair[np.arange(T) * k + j]
    if dims.n_shared:
        dxo += dx_pair[P:P + T]
    out = {"dx": dxo, "dx_pair": dx_pair}
    out.update(grads)
    return out


def backward_tokens(inp, topk_ids, topk_w, dims, tokens, dtype=np.float64):
    """dX rows for the listed tokens only."""
    n, k, s = dims.n, dims.k, dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    dY = decode(inp, "dy", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    ids = np.asarray(topk_ids)
    out = np.zeros((len(tokens), dims.d), dtype)
    for i, t in enumerate(tokens):
        xt, dyt = X[t:t + 1], dY[t:t + 1]
        for j in range(k):
            out[i] += _expert_backward(xt, w[t, j] * dyt, W, int(ids[t, j]), n, s)[0][0]
        for e in range(dims.E, dims.E_tot):
            out[i] += _expert_backward(xt, dyt, W, e, n, s)[0][0]
    return out


def lora_grads_expert(inp, topk_ids, topk_w, dims, e, dtype=np.float64):
    """(dA_gu, dB_gu, dA_dn, dB_dn) of one expert, from all of its rows."""
    T, k, n, s = dims.T, dims.k, dims.n, dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    dY = decode(inp, "dy", dtype)
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    if e < dims.E:
        tok, slot = np.nonzero(np.asarray(topk_ids) == e)
        wt = w[tok, slot][:, None]
    else:
        tok, wt = np.arange(T), 1.0
    if tok.size == 0:
        return (np.zeros((dims.d, dims.r), dtype), np.zeros((dims.r, 2 * n), dtype),
                np.zeros((n, dims.r), dtype), np.zeros((dims.r, dims.d), dtype))
    return _expert_backward(X[tok], wt * dY[tok], W, e, n, s)[1:]


# ----------------------------------------------------------------------------
# Gradients that reach the router (beyond the pages' frozen router)
# ----------------------------------------------------------------------------

def router_grads(inp, topk_ids, topk_w, dims, dtype=np.float64, fw=None):
    """Routing-weight and logit gradients of the layer, given dY (``inp.dy``).

    Y[t] is linear in the routing weights, so
      d_topk_w[t, j] = <dY[t], O(t, expert j)>;
    w[t, :] is the softmax of the k selected logits, whose Jacobian is
    dw_j / dl_i = w_j (delta_ij - w_i), so
      d_logits[t, ids[t, i]] = w[t, i] (d_topk_w[t, i] - sum_j w[t, j] d_topk_w[t, j]),
    and the logits of experts not selected get 0 (a small change leaves the
    selection as it is).  The shared expert's weight is the constant 1.
    ``fw`` may pass the result of ``forward`` on the same arguments, whose
    per-pair outputs O are then reused.
    """
    T, k = dims.T, dims.k
    if fw is None:
        fw = forward(inp, topk_ids, topk_w, dims, dtype)
    dY = decode(inp, "dy", dtype)
    o = fw["o_pair"][:T * k].reshape(T, k, dims.d)
    dw = (dY[:, None, :] * o).sum(axis=2)
    return _softmax_topk_backward(dw, topk_ids, topk_w, dims.E, dtype)


def _softmax_topk_backward(dw, topk_ids, topk_w, E, dtype):
    w = np.asarray(topk_w, dtype=np.float32).astype(dtype)
    dsel = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    dl = np.zeros((dw.shape[0], E), dtype)
    dl[np.arange(dw.shape[0])[:, None], np.asarray(topk_ids, dtype=np.int64)] = dsel
    return {"d_topk_w": dw, "d_logits": dl}


def router_grads_tokens(inp, topk_ids, topk_w, dims, tokens, dtype=np.float64):
    """``router_grads`` rows for the listed tokens only (each from its own k
    pairs, as ``forward_tokens``)."""
    n, k, s = dims.n, dims.k, dims.lora_scale
    W = _params(inp, dtype)
    X = decode(inp, "x", dtype)
    dY = decode(inp, "dy", dtype)
    ids = np.asarray(topk_ids)
    dw = np.zeros((len(tokens), k), dtype)
    for i, t in enumerate(tokens):
        for j in range(k):
            o = expert_forward(X[t:t + 1], W, int(ids[t, j]), n, s)[2][0]
            dw[i, j] = np.sum(dY[t] * o)
    tk = np.asarray(tokens)
    return _softmax_topk_backward(dw, ids[tk], np.asarray(topk_w)[tk], dims.E, dtype)
