"""CPU oracle of the dropless top-k Mixture-of-Experts SwiGLU FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's ``smoke()`` check and
the ``cpu_baseline`` leg of the benchmark may import this module.  It shares
no code with the HIP path and the HIP path never calls it.

The layer computes, for every token x_n (a row of x [N, H]):

    y_n = sum_k g_{n,k} * FFN_{e_{n,k}}(x_n)

with router logits l = x.W_r (+ b), the K experts e_{n,0..K-1} of largest
logit, renormalised gates g, and SwiGLU experts
FFN_e(v) = (silu(v.W_gate[e]) * (v.W_up[e])).W_down[e].

Sources (page titles; the text of each page is what is followed):
  * "MoE computation principle and execution process: from Router scoring to
    expert parallelism and load balancing" (icman.com.cn): section 2.1 (router
    logits x.W_r with W_r [H, E]), 2.2 (softmax, top-K, renormalise the K
    selected weights; gradient only through the continuous weights), 2.3
    (SwiGLU expert silu(gate) * up then down projection; weighted sum over the
    K selected experts), 2.4 (tiny example shapes and init).
  * "MoE technical analysis: from theory to practice" (intelliparadigm.com):
    section 2.1 (SwiGLU FeedForward without biases, silu on the w1 branch),
    2.3 (top-k on the gate logits, softmax over the K values, per-expert loop
    with an index_add_ combine).
  * "MegaBlocks - architecture and principles" (ai-reference-codex): section
    2.1 / 2.3 (dropless metadata: sort by expert, histogram, cumsum into bins;
    gather, expert MLP, weighted scatter with a top-k sum), section 4 (sort
    only on the expert-id key; gather and scatter are each other's backward).
  * "MoK: high-performance Megakernel for deterministic training of large MoE
    models" (jsqmd.com): section 3.1/3.3 (gating, top-k, index_add combine),
    section 4.3 and 6.2 (deterministic top-k and sort, identical reruns).
  * "MoonEP: how Moonshot AI solved the imbalance problem in MoE models"
    (aikraft.ru): section 01 (the maxvio skew metric).

Readings where the pages are silent or ambiguous (each also listed in the
design notes of the repository):
  * top-K is taken on the logits with the order (logit descending, expert id
    ascending); slot k of a token is its rank in that order;
  * gates are the softmax over the K selected logits, which equals the full
    softmax renormalised over the K selected experts;
  * sorting by expert is stable in the flat index f = n*K + k;
  * no bias in the experts; the optional logit bias b [E] is a constant input
    that changes both selection and gate values and gets no gradient;
  * weights are stored for x.W: W_gate, W_up [E, H, F], W_down [E, F, H];
  * unselected router logits get exactly zero gradient.

Precision.  All arithmetic is float64.  ``store`` selects where values are
rounded, to mirror the storage precision of a device implementation:
  * "f64": no rounding (exact mode);
  * "f32": every tensor that is stored between steps is rounded to float32;
  * "bf16": every activation tensor stored between steps (xs, G, U, A, ys, y,
    dys, dG, dU, dxs, dx) is rounded to bfloat16 with round-to-nearest-even;
    gates, dgates and dlogits are rounded to float32; logits, the expert
    partial sums and all weight gradients stay float64.

Parity pins: see tests/test_oracle_pins.py (brute-force per-token
evaluation, library routines for the metadata, closed-form special cases,
central finite differences, and autograd of an independent dense-masked
formulation).
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

STORE_TYPES = ("f64", "f32", "bf16")


# --------------------------------------------------------------------------
# rounding helpers
# --------------------------------------------------------------------------

def as_f64(a) -> np.ndarray:
    """Convert a torch tensor (any float dtype) or array to a float64 ndarray."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        if str(a.dtype) in ("torch.bfloat16", "torch.float16"):
            import torch
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps the sign, the 8-bit exponent and the top 7 mantissa bits
    of a float32; in float64 terms it keeps the top 7 of 52 mantissa bits,
    so the low 45 bits are rounded away.
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    u = a.view(np.uint64)
    keep_lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + keep_lsb) & ~((np.uint64(1) << np.uint64(45)) - np.uint64(1))
    out = r.view(np.float64)
    # values beyond the bfloat16 range become +-inf, as a float32 cast would
    return out.astype(np.float32).astype(np.float64)


def rho(a: np.ndarray, store: str) -> np.ndarray:
    """Storage rounding of an activation tensor."""
    if store == "f64":
        return a
    if store == "f32":
        return a.astype(np.float32).astype(np.float64)
    if store == "bf16":
        return round_bf16(a)
    raise ValueError(store)


def rho32(a: np.ndarray, store: str) -> np.ndarray:
    """Storage rounding of a tensor kept in float32 (gates and router grads)."""
    if store == "f64":
        return a
    return a.astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# router (icman 2.1, 2.2; intelliparadigm 2.3)
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits l = x.W_r (+ b): one score per (token, expert)."""
    l = x @ w_r
    if bias is not None:
        l = l + bias[None, :]
    return l


def topk_experts(logits: np.ndarray, K: int) -> np.ndarray:
    """The K experts of largest logit per token, ordered (logit desc, id asc).

    A stable sort of the negated logits keeps equal logits in ascending
    expert-id order, which is the tie-break.
    """
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :K]).astype(np.int32)


def gates_topk_softmax(logits: np.ndarray, topk: np.ndarray) -> np.ndarray:
    """Gates as the softmax over the K selected logits (intelliparadigm 2.3)."""
    sel = np.take_along_axis(logits, topk.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def gates_renormalised_softmax(logits: np.ndarray, topk: np.ndarray) -> np.ndarray:
    """Gates as the full softmax over E renormalised over the K selected (icman 2.2)."""
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, topk.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# dropless routing metadata (MegaBlocks 2.1 / 2.3, section 4)
# --------------------------------------------------------------------------

def routing_metadata(topk: np.ndarray, E: int, capacity: Optional[int] = None):
    """Histogram, cumsum bins and the stable sort of the flat assignment.

    Returns (counts [E], offsets [E+1], sorted_flat [NK], inv [NK]) where
    offsets is the exclusive cumsum of counts (offsets[1:] are the inclusive
    bins), sorted_flat[i] is the flat index f = n*K + k of the i-th row of
    the expert-grouped order (stable in f), and inv[f] is the row of f.

    With a capacity C ("MoE computation principle and execution process",
    section 3.4: each expert takes at most C rows, the overflow is dropped),
    expert e keeps the first min(counts[e], C) of its rows in that stable
    order (the lowest flat indices).  counts stays the full histogram of the
    assignment; offsets bins the kept rows only; sorted_flat holds the kept
    rows, expert-grouped, followed by -1 for every dropped row; inv[f] is -1
    for a dropped f.
    """
    flat = topk.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable").astype(np.int64)
    start = np.zeros(E + 1, dtype=np.int64)
    start[1:] = np.cumsum(counts)
    rank = np.arange(order.size, dtype=np.int64) - start[flat[order]]   # position within the expert
    keep = np.ones(order.size, dtype=bool) if capacity is None else rank < capacity
    kept_counts = counts if capacity is None else np.minimum(counts, capacity)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_counts)
    sorted_flat = np.full(order.size, -1, dtype=np.int64)
    sorted_flat[:int(offsets[E])] = order[keep]
    inv = np.full(order.size, -1, dtype=np.int64)
    inv[order[keep]] = np.arange(int(offsets[E]), dtype=np.int64)
    return counts, offsets, sorted_flat, inv


def capacity_of(N: int, K: int, E: int, capacity_factor: float) -> int:
    """Expert capacity ceil(capacity_factor * N * K / E): the page's
    ceil(N / E * capacity_factor) with N read as the N * K routed slots
    ("MoE computation principle and execution process", section 3.4)."""
    return int(math.ceil(capacity_factor * N * K / E))


def tile_list(counts: np.ndarray, offsets: np.ndarray, tile_m: int) -> np.ndarray:
    """Row tiles of the grouped GEMM: (expert, first row, rows) per tile.

    Experts ascending; each expert's rows [offsets[e], offsets[e+1]) are cut
    into ceil(counts[e] / tile_m) tiles of tile_m rows, the last one ragged.
    Padding exists only as tile granularity, never in memory.
    """
    tiles = []
    for e in range(counts.size):
        c = int(counts[e])
        t = 0
        while t * tile_m < c:
            tiles.append((e, int(offsets[e]) + t * tile_m, min(tile_m, c - t * tile_m)))
            t += 1
    return np.asarray(tiles, dtype=np.int64).reshape(-1, 3)


def maxvio(counts: np.ndarray, N: int, K: int, E: int) -> float:
    """max_e(T_e / T_bar) - 1 with T_bar = N*K/E (MoonEP section 01)."""
    tbar = N * K / E
    return float(np.max(counts) / tbar - 1.0)


# --------------------------------------------------------------------------
# SwiGLU expert (icman 2.3; intelliparadigm 2.1)
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_expert(xs: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, store: str):
    """One expert on its rows: G = xs.Wg, U = xs.Wu, A = silu(G)*U, ys = A.Wd."""
    G = rho(xs @ wg, store)
    U = rho(xs @ wu, store)
    A = rho(silu(G) * U, store)
    ys = rho(A @ wd, store)
    return G, U, A, ys


# --------------------------------------------------------------------------
# Switch load-balancing loss (icman 4.2)
# --------------------------------------------------------------------------
#
# L_aux = alpha * E * sum_i f_i * P_i with f_i the share of the N*K routed
# assignments that went to expert i (counts_i / (N*K); the token share for
# K = 1) and P_i the router's softmax probability of expert i averaged over
# all N tokens, from the same logits that select the experts (bias
# included).  f is a count and carries no gradient.

def router_probs(logits: np.ndarray) -> np.ndarray:
    """Softmax over all E experts of every token's logits."""
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def aux_loss(logits: np.ndarray, counts: np.ndarray, K: int, alpha: float) -> float:
    """alpha * E * sum_i f_i P_i."""
    N, E = logits.shape
    P = router_probs(logits).mean(axis=0)
    f = np.asarray(counts, dtype=np.float64) / (N * K)
    return float(alpha * E * np.sum(f * P))


def aux_loss_grad(logits: np.ndarray, counts: np.ndarray, K: int, scale: float) -> np.ndarray:
    """d(L_aux)/d logits with alpha * (upstream gradient) = scale:
    scale * E / N * p[n,j] * (f_j - sum_i f_i p[n,i]) (P_j is the mean of the
    p[n,j], whose softmax derivative is p[n,j] (delta_ij - p[n,i]))."""
    N, E = logits.shape
    p = router_probs(logits)
    f = np.asarray(counts, dtype=np.float64) / (N * K)
    s = p @ f
    return scale * E / N * p * (f[None, :] - s[:, None])


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def forward(x, w_r, w_gate, w_up, w_down, K: int, bias=None, store: str = "bf16", tile_m: int = 128,
            topk=None, capacity: Optional[int] = None, shared=None):
    """Forward pass of the layer; returns every intermediate in a dict.

    Steps in the pages' order: logits, top-K, gates, metadata (histogram,
    cumsum, stable sort), gather, per-expert SwiGLU on the expert's rows,
    gate-weighted index_add combine back to token order.

    ``topk`` [N, K] (optional) replaces the top-K selection with a given
    assignment of K distinct experts per token, in slot order, for checks
    made "given the same assignment"; the gates are still the softmax over
    the logits of the given experts.

    ``capacity`` (optional) caps the rows each expert takes (see
    routing_metadata); a dropped slot contributes nothing to y and its gate
    is not renormalised away.  Rows past the kept ones stay zero.

    ``shared`` (optional) = (W_gate_s [H,Fs], W_up_s [H,Fs], W_down_s [Fs,H]):
    a dense SwiGLU expert every token passes through with weight 1, added to
    the routed output ("MegaBlocks - architecture and principles", section
    2.1: the layer's output plus an optional shared-expert MLP over all
    tokens): y = round(sum_k g_k ys[inv] + ys_s), ys_s stored rounded.
    """
    assert store in STORE_TYPES
    x = as_f64(x)
    w_r = as_f64(w_r)
    bias = as_f64(bias)
    wg_all, wu_all, wd_all = as_f64(w_gate), as_f64(w_up), as_f64(w_down)
    N, H = x.shape
    E = w_r.shape[1]
    F = wg_all.shape[2]

    logits = router_logits(x, w_r, bias)
    if topk is None:
        topk = topk_experts(logits, K)
    else:
        topk = np.ascontiguousarray(np.asarray(topk).reshape(N, K)).astype(np.int32)
        assert all(len(set(r.tolist())) == K for r in topk), "a token's experts must be distinct"
        assert topk.min() >= 0 and topk.max() < E
    gates = rho32(gates_topk_softmax(logits, topk), store)
    counts, offsets, sorted_flat, inv = routing_metadata(topk, E, capacity)
    tiles = tile_list(np.diff(offsets), offsets, tile_m)

    NK = N * K
    nkept = int(offsets[E])
    tok = np.maximum(sorted_flat, 0) // K
    xs = np.zeros((NK, H))
    xs[:nkept] = x[tok[:nkept]]
    G = np.zeros((NK, F))
    U = np.zeros((NK, F))
    A = np.zeros((NK, F))
    ys = np.zeros((NK, H))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        G[r0:r1], U[r0:r1], A[r0:r1], ys[r0:r1] = swiglu_expert(xs[r0:r1], wg_all[e], wu_all[e], wd_all[e], store)

    # shared expert: every token, token order, weight 1
    sh = None
    if shared is not None:
        wgs, wus, wds = (as_f64(w) for w in shared)
        Gs, Us, As, yss = swiglu_expert(x, wgs, wus, wds, store)
        sh = dict(w_gate=wgs, w_up=wus, w_down=wds, G=Gs, U=Us, A=As, ys=yss)

    # index_add-style combine: each expert adds its gate-weighted rows into
    # the tokens they came from
    y = np.zeros((N, H))
    gflat = gates.reshape(-1)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        f = sorted_flat[r0:r1]
        np.add.at(y, f // K, gflat[f][:, None] * ys[r0:r1])
    if sh is not None:
        y = y + sh["ys"]
    y = rho(y, store)
    return dict(x=x, w_r=w_r, bias=bias, w_gate=wg_all, w_up=wu_all, w_down=wd_all, K=K, store=store,
                logits=logits, topk=topk, gates=gates, counts=counts, offsets=offsets,
                sorted_flat=sorted_flat, inv=inv, tiles=tiles, xs=xs, G=G, U=U, A=A, ys=ys, y=y,
                capacity=capacity, shared=sh)


def backward(fwd: dict, dy, aux_scale: Optional[float] = None) -> dict:
    """Backward pass given the forward intermediates and dL/dy.

    With aux_scale (alpha times the upstream gradient of the load-balancing
    loss), the gradient of that loss is added to dlogits before the router's
    weight and input gradients are formed.

    combine backward (gather of dy weighted by the gate, and the gate
    gradient as a dot product), expert backward with the SwiGLU derivative,
    router backward through the softmax over the selected logits only, and
    the gather backward (sum of the K rows of each token) plus the router's
    input gradient.
    """
    store = fwd["store"]
    K = fwd["K"]
    dy = as_f64(dy)
    x, w_r = fwd["x"], fwd["w_r"]
    N, H = x.shape
    E = w_r.shape[1]
    F = fwd["w_gate"].shape[2]
    NK = N * K
    sorted_flat, inv, offsets = fwd["sorted_flat"], fwd["inv"], fwd["offsets"]
    gates, topk = fwd["gates"], fwd["topk"]
    gflat = gates.reshape(-1)
    kept_row = sorted_flat >= 0                            # rows past the kept ones: dropped slots
    sf = np.maximum(sorted_flat, 0)
    tok = sf // K
    kept_slot = (inv >= 0).reshape(N, K)

    # combine backward (a dropped slot has no row and a zero gate gradient)
    dys = rho(np.where(kept_row[:, None], gflat[sf][:, None] * dy[tok], 0.0), store)
    ys_tok = fwd["ys"][np.maximum(inv, 0).reshape(N, K)] * kept_slot[:, :, None]   # [N, K, H]
    dgates = rho32(np.einsum("nh,nkh->nk", dy, ys_tok), store)

    # expert backward
    dG = np.zeros((NK, F))
    dU = np.zeros((NK, F))
    dxs = np.zeros((NK, H))
    dw_gate = np.zeros_like(fwd["w_gate"])
    dw_up = np.zeros_like(fwd["w_up"])
    dw_down = np.zeros_like(fwd["w_down"])
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        G, U, A = fwd["G"][r0:r1], fwd["U"][r0:r1], fwd["A"][r0:r1]
        xs = fwd["xs"][r0:r1]
        d = dys[r0:r1]
        dA = d @ fwd["w_down"][e].T
        sg = sigmoid(G)
        dG[r0:r1] = rho(dA * U * sg * (1.0 + G * (1.0 - sg)), store)
        dU[r0:r1] = rho(dA * (G * sg), store)
        dxs[r0:r1] = rho(dG[r0:r1] @ fwd["w_gate"][e].T + dU[r0:r1] @ fwd["w_up"][e].T, store)
        dw_gate[e] = xs.T @ dG[r0:r1]
        dw_up[e] = xs.T @ dU[r0:r1]
        dw_down[e] = A.T @ d

    # router backward: only the selected logits receive a gradient
    s = np.sum(gates * dgates, axis=1, keepdims=True)
    dsel = gates * (dgates - s)
    dlogits = np.zeros((N, E))
    np.put_along_axis(dlogits, topk.astype(np.int64), dsel, axis=1)
    if aux_scale is not None:
        dlogits = dlogits + aux_loss_grad(fwd["logits"], fwd["counts"], K, aux_scale)
    dlogits = rho32(dlogits, store)

    # shared expert backward: its upstream gradient is dy itself
    out_sh = {}
    sh = fwd.get("shared")
    if sh is not None:
        dA = dy @ sh["w_down"].T
        sg = sigmoid(sh["G"])
        dGs = rho(dA * sh["U"] * sg * (1.0 + sh["G"] * (1.0 - sg)), store)
        dUs = rho(dA * (sh["G"] * sg), store)
        dxs_s = rho(dGs @ sh["w_gate"].T + dUs @ sh["w_up"].T, store)
        out_sh = dict(dG_s=dGs, dU_s=dUs, dxs_s=dxs_s, dw_gate_s=x.T @ dGs, dw_up_s=x.T @ dUs,
                      dw_down_s=sh["A"].T @ dy)

    # gather backward (sum over each token's kept rows) + router input
    # gradient (+ the shared expert's input gradient)
    dx = (dxs[np.maximum(inv, 0).reshape(N, K)] * kept_slot[:, :, None]).sum(axis=1) + dlogits @ w_r.T
    if sh is not None:
        dx = dx + out_sh["dxs_s"]
    dx = rho(dx, store)
    dw_r = x.T @ dlogits
    return dict(dys=dys, dgates=dgates, dG=dG, dU=dU, dxs=dxs, dlogits=dlogits, dx=dx, dw_r=dw_r,
                dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down, **out_sh)


# --------------------------------------------------------------------------
# one token at a time (for sampled checks at sizes where the whole layer is
# too slow on the CPU)
# --------------------------------------------------------------------------

ExpertFn = Callable[[int], tuple]


def token_forward(xn, w_r, bias, expert_weights: ExpertFn, K: int, store: str = "bf16") -> dict:
    """Forward of one token: its K experts, gates, expert rows and output.

    ``expert_weights(e)`` returns (W_gate[e], W_up[e], W_down[e]).
    """
    xn = as_f64(xn).reshape(1, -1)
    l = router_logits(xn, as_f64(w_r), as_f64(bias))
    top = topk_experts(l, K)
    g = rho32(gates_topk_softmax(l, top), store)[0]
    rows = []
    y = np.zeros(xn.shape[1])
    for k in range(K):
        wg, wu, wd = (as_f64(w) for w in expert_weights(int(top[0, k])))
        G, U, A, ys = swiglu_expert(xn, wg, wu, wd, store)
        rows.append(dict(G=G[0], U=U[0], A=A[0], ys=ys[0]))
        y = y + g[k] * ys[0]
    return dict(logits=l[0], topk=top[0], gates=g, rows=rows, y=rho(y, store))


def token_backward(tf: dict, dyn, w_r, expert_weights: ExpertFn, store: str = "bf16") -> dict:
    """Backward of one token given its token_forward result and dL/dy_n.

    Every quantity here depends on the token alone: dys, dgates, the expert
    row gradients dG, dU, dxs, the router gradient and dx_n.
    """
    dyn = as_f64(dyn).reshape(-1)
    w_r = as_f64(w_r)
    K = tf["topk"].size
    g = tf["gates"]
    dg = np.zeros(K)
    dxs_sum = np.zeros_like(dyn)
    out_rows = []
    for k in range(K):
        r = tf["rows"][k]
        dg[k] = float(dyn @ r["ys"])
        wg, wu, wd = (as_f64(w) for w in expert_weights(int(tf["topk"][k])))
        dys = rho(g[k] * dyn, store)
        dA = dys @ wd.T
        G, U = r["G"], r["U"]
        sg = sigmoid(G)
        dG = rho(dA * U * sg * (1.0 + G * (1.0 - sg)), store)
        dU = rho(dA * (G * sg), store)
        dxs = rho(dG @ wg.T + dU @ wu.T, store)
        dxs_sum = dxs_sum + dxs
        out_rows.append(dict(dys=dys, dG=dG, dU=dU, dxs=dxs))
    dg = rho32(dg, store)
    s = float(np.sum(g * dg))
    dsel = rho32(g * (dg - s), store)
    dl = np.zeros(w_r.shape[1])
    dl[tf["topk"].astype(np.int64)] = dsel
    dx = rho(dxs_sum + w_r @ dl, store)
    return dict(dgates=dg, dlogits=dl, rows=out_rows, dx=dx)


# --------------------------------------------------------------------------
# rounding-decision bands (bf16 storage)
# --------------------------------------------------------------------------
#
# A device implementation accumulates in float32, so the value it rounds to
# bfloat16 differs from the exact value by a few float32 roundings.  Where the
# exact value lies that close to a rounding midpoint, either neighbouring
# bfloat16 value is a correct result, and the choice propagates into later
# sums.  rounding_bands() returns, per element of each bf16-stored tensor, a
# first-order bound of the deviation such choices can cause, capped at two
# bf16 spacings of the element (of the element and the K rows summed into it,
# for y and dx); it is zero wherever no rounding decision upstream of the
# element was ambiguous.  Tests compare |device - oracle| <= tolerance + band,
# which checks every unique result exactly and every ambiguous one for
# validity.  The float32 outputs (dgates, dlogits, the weight gradients) get
# no band: they sum bf16-stored values over H or over thousands of tokens, so
# the flips of two correct runs add up there, and they are checked step by
# step from the run's own stored inputs instead.

BAND_CAP_SPACINGS = 2.0


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Distance from the bfloat16 value v to the next one away from zero
    (2^(e - 7) for |v| in [2^e, 2^(e+1))); 0 at v = 0."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)

U32 = 2.0 ** -24  # unit roundoff of float32


def gemm_sigma(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Bound of the float32 accumulation error of a @ b (exact products,
    n-term sums): 4 u sqrt(n) ||row_a * col_b||_2 + 4 u |a @ b|."""
    n = a.shape[-1]
    return 4 * U32 * math.sqrt(max(n, 1)) * np.sqrt((a * a) @ (b * b)) + 4 * U32 * np.abs(a @ b)


def bf16_flip(pre: np.ndarray, rounded: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """Deviation bound of a bfloat16 rounding whose input is known to within
    +-sigma: sigma + the spacing to the other candidate where the interval
    reaches a rounding midpoint, else 0 (both ends round alike)."""
    r32 = np.ascontiguousarray(rounded, dtype=np.float32)
    bits = r32.view(np.uint32).astype(np.int64)
    diff = pre - rounded
    away = (np.sign(diff) == np.sign(rounded)) & (diff != 0)
    nb_bits = np.where(away, bits + 0x10000, bits - 0x10000) & 0xFFFFFFFF
    nb = nb_bits.astype(np.uint32).view(np.float32).astype(np.float64)
    spacing = np.where(rounded == 0, 0.0, np.abs(nb - rounded))
    dist = spacing / 2 - np.abs(diff)
    return np.where(dist <= sigma, sigma + spacing, 0.0)


def _silu_d1(g):
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def _silu_d2(g):
    s = sigmoid(g)
    return s * (1.0 - s) * (2.0 + g * (1.0 - 2.0 * s))


def prop(dev: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Deviation of dev-perturbed rows multiplied by w (dev @ w): the smaller of
    the worst case |dev| @ |w| and four standard deviations of a sum of
    independent-sign terms, 4 sqrt(dev^2 @ w^2)."""
    return np.minimum(dev @ np.abs(w), 4.0 * np.sqrt((dev * dev) @ (w * w)))


def rounding_bands(fwd: dict, bwd: Optional[dict] = None, dy=None, aux_scale: Optional[float] = None,
                   cap: bool = True) -> dict:
    """Per-element deviation bounds (see above) of every bf16-stored tensor
    of a bf16-storage forward (and backward, with the load-balancing loss
    gradient when aux_scale is given) computed by this module, each capped
    at BAND_CAP_SPACINGS bf16 spacings."""
    assert fwd["store"] == "bf16"
    K = fwd["K"]
    x, w_r = fwd["x"], fwd["w_r"]
    N, H = x.shape
    E = w_r.shape[1]
    NK = N * K
    F = fwd["w_gate"].shape[2]
    off, sf, inv = fwd["offsets"], fwd["sorted_flat"], fwd["inv"]
    # dropped slots (capacity) have no row: masked out of every sum below
    kept2 = (inv >= 0).reshape(N, K)
    kept_row = (sf >= 0)[:, None]
    inv2 = np.maximum(inv, 0).reshape(N, K)
    tok = np.maximum(sf, 0) // K
    gflat = fwd["gates"].reshape(-1)
    grow = gflat[np.maximum(sf, 0)][:, None] * kept_row
    xs, G, U, A, ys = fwd["xs"], fwd["G"], fwd["U"], fwd["A"], fwd["ys"]
    b = {k: np.zeros((NK, F)) for k in ("G", "U", "A")}
    b["ys"] = np.zeros((NK, H))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        sl = slice(r0, r1)
        wg, wu, wd = fwd["w_gate"][e], fwd["w_up"][e], fwd["w_down"][e]
        b["G"][sl] = bf16_flip(xs[sl] @ wg, G[sl], gemm_sigma(xs[sl], wg))
        b["U"][sl] = bf16_flip(xs[sl] @ wu, U[sl], gemm_sigma(xs[sl], wu))
        ap = silu(G[sl]) * U[sl]
        sa = np.abs(U[sl] * _silu_d1(G[sl])) * b["G"][sl] + np.abs(silu(G[sl])) * b["U"][sl] + 16 * U32 * np.abs(ap)
        b["A"][sl] = bf16_flip(ap, A[sl], sa)
        b["ys"][sl] = bf16_flip(A[sl] @ wd, ys[sl], gemm_sigma(A[sl], wd) + prop(b["A"][sl], wd))
    yp = np.zeros((N, H))
    sy = np.zeros((N, H))
    sh = fwd.get("shared")
    if sh is not None:
        # shared expert: one more expert over all tokens (rows = x), weight 1
        Gs, Us, As, yss = sh["G"], sh["U"], sh["A"], sh["ys"]
        b["G_s"] = bf16_flip(x @ sh["w_gate"], Gs, gemm_sigma(x, sh["w_gate"]))
        b["U_s"] = bf16_flip(x @ sh["w_up"], Us, gemm_sigma(x, sh["w_up"]))
        ap = silu(Gs) * Us
        sa = np.abs(Us * _silu_d1(Gs)) * b["G_s"] + np.abs(silu(Gs)) * b["U_s"] + 16 * U32 * np.abs(ap)
        b["A_s"] = bf16_flip(ap, As, sa)
        b["ys_s"] = bf16_flip(As @ sh["w_down"], yss, gemm_sigma(As, sh["w_down"]) + prop(b["A_s"], sh["w_down"]))
        yp += yss
        sy += b["ys_s"] + 8 * U32 * np.abs(yss)
    for k in range(K):
        r = inv2[:, k]
        g = fwd["gates"][:, k:k + 1] * kept2[:, k:k + 1]
        yp += g * ys[r]
        sy += g * b["ys"][r] + 8 * U32 * np.abs(g * ys[r])
    b["y"] = bf16_flip(yp, fwd["y"], sy)
    if bwd is None:
        return _capped(b, fwd, None, cap)

    dy = as_f64(dy)
    # combine backward
    dysp = grow * dy[tok]
    b["dys"] = bf16_flip(dysp, bwd["dys"], 8 * U32 * np.abs(dysp))
    ys_tok = ys[inv2] * kept2[:, :, None]
    b_ys_tok = b["ys"][inv2] * kept2[:, :, None]
    lin = np.einsum("nh,nkh->nk", np.abs(dy), b_ys_tok)
    rss = 4.0 * np.sqrt(np.einsum("nh,nkh->nk", dy * dy, b_ys_tok * b_ys_tok))
    b["dgates"] = (np.minimum(lin, rss)
                   + 4 * U32 * math.sqrt(H) * np.sqrt(np.einsum("nh,nkh->nk", dy * dy, ys_tok * ys_tok))
                   + 2 * U32 * np.abs(bwd["dgates"]))
    # expert backward
    for k in ("dG", "dU"):
        b[k] = np.zeros((NK, F))
    b["dxs"] = np.zeros((NK, H))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        sl = slice(r0, r1)
        wg, wu, wd = fwd["w_gate"][e], fwd["w_up"][e], fwd["w_down"][e]
        d = bwd["dys"][sl]
        dA = d @ wd.T
        sdA = gemm_sigma(d, wd.T) + prop(b["dys"][sl], wd.T)
        g_, u_ = G[sl], U[sl]
        d1, d2 = _silu_d1(g_), _silu_d2(g_)
        dgp = dA * u_ * d1
        sdg = (np.abs(u_ * d1) * sdA + np.abs(dA * d1) * b["U"][sl] + np.abs(dA * u_ * d2) * b["G"][sl]
               + 16 * U32 * np.abs(dgp))
        b["dG"][sl] = bf16_flip(dgp, bwd["dG"][sl], sdg)
        dup = dA * silu(g_)
        sdu = np.abs(silu(g_)) * sdA + np.abs(dA * d1) * b["G"][sl] + 16 * U32 * np.abs(dup)
        b["dU"][sl] = bf16_flip(dup, bwd["dU"][sl], sdu)
        dG, dU = bwd["dG"][sl], bwd["dU"][sl]
        dxp = dG @ wg.T + dU @ wu.T
        sdx = gemm_sigma(dG, wg.T) + gemm_sigma(dU, wu.T) + prop(b["dG"][sl], wg.T) + prop(b["dU"][sl], wu.T)
        b["dxs"][sl] = bf16_flip(dxp, bwd["dxs"][sl], sdx)
    # router backward
    g = fwd["gates"]
    sdl = g * (b["dgates"] + np.sum(g * b["dgates"], axis=1, keepdims=True)) + 8 * U32 * (
        np.abs(g * bwd["dgates"]) + g * np.sum(np.abs(g * bwd["dgates"]), axis=1, keepdims=True))
    b["dlogits"] = np.zeros((N, E))
    np.put_along_axis(b["dlogits"], fwd["topk"].astype(np.int64), sdl, axis=1)
    if aux_scale is not None:
        # float32 logits are within gemm_sigma of the exact ones; the aux term
        # p (f - s) moves by at most 4 max(f) p per unit of logit change, plus
        # a few float32 roundings of the softmax and the products
        aux = aux_loss_grad(fwd["logits"], fwd["counts"], K, aux_scale)
        dl_max = gemm_sigma(x, w_r).max(axis=1, keepdims=True)
        p = router_probs(fwd["logits"])
        fmax = float(np.max(fwd["counts"])) / NK
        b["dlogits"] = b["dlogits"] + 64 * U32 * np.abs(aux) + (
            abs(aux_scale) * E / N * p * 4 * fmax * dl_max + 8 * U32 * np.abs(bwd["dlogits"]))
    # gather backward
    dxs_tok = bwd["dxs"][inv2] * kept2[:, :, None]
    dxp = dxs_tok.sum(axis=1) + bwd["dlogits"] @ w_r.T
    sdx = ((b["dxs"][inv2] * kept2[:, :, None]).sum(axis=1) + prop(b["dlogits"], w_r.T)
           + 8 * U32 * (np.abs(dxs_tok).sum(axis=1) + np.abs(bwd["dlogits"]) @ np.abs(w_r.T)))
    if sh is not None:
        # shared expert backward (its dys is dy itself, exact)
        Gs, Us, As = sh["G"], sh["U"], sh["A"]
        dA = dy @ sh["w_down"].T
        sdA = gemm_sigma(dy, sh["w_down"].T)
        d1, d2 = _silu_d1(Gs), _silu_d2(Gs)
        dgp = dA * Us * d1
        b["dG_s"] = bf16_flip(dgp, bwd["dG_s"], np.abs(Us * d1) * sdA + np.abs(dA * d1) * b["U_s"]
                              + np.abs(dA * Us * d2) * b["G_s"] + 16 * U32 * np.abs(dgp))
        dup = dA * silu(Gs)
        b["dU_s"] = bf16_flip(dup, bwd["dU_s"], np.abs(silu(Gs)) * sdA + np.abs(dA * d1) * b["G_s"]
                              + 16 * U32 * np.abs(dup))
        dGs, dUs = bwd["dG_s"], bwd["dU_s"]
        dxsp = dGs @ sh["w_gate"].T + dUs @ sh["w_up"].T
        b["dxs_s"] = bf16_flip(dxsp, bwd["dxs_s"], gemm_sigma(dGs, sh["w_gate"].T) + gemm_sigma(dUs, sh["w_up"].T)
                               + prop(b["dG_s"], sh["w_gate"].T) + prop(b["dU_s"], sh["w_up"].T))
        dxp = dxp + bwd["dxs_s"]
        sdx = sdx + b["dxs_s"] + 8 * U32 * np.abs(bwd["dxs_s"])
    b["dx"] = bf16_flip(dxp, bwd["dx"], sdx)
    return _capped(b, fwd, bwd, cap)


def _capped(b: dict, fwd: dict, bwd: Optional[dict], cap: bool = True) -> dict:
    """The bands of the bf16-stored tensors, each at most BAND_CAP_SPACINGS
    spacings of the element; for y and dx the spacings of the K rows (and
    the shared expert's row) summed into the element count as well."""
    c = BAND_CAP_SPACINGS if cap else np.inf
    vals = dict(fwd)
    if bwd is not None:
        vals.update(bwd)
    sh = fwd.get("shared")
    if sh is not None:
        vals.update({k + "_s": sh[k] for k in ("G", "U", "A", "ys")})
    N, K = fwd["gates"].shape
    inv = fwd["inv"].reshape(N, K)
    kept = (inv >= 0)[:, :, None]
    rows = np.maximum(inv, 0)
    out = {}
    for name in ("G", "U", "A", "ys", "dys", "dG", "dU", "dxs", "G_s", "U_s", "A_s", "ys_s", "dG_s", "dU_s", "dxs_s"):
        if name in b and name in vals:
            out[name] = np.minimum(b[name], c * bf16_spacing(vals[name]))
    cap_y = bf16_spacing(fwd["y"]) + (fwd["gates"][:, :, None] * bf16_spacing(fwd["ys"])[rows] * kept).sum(axis=1)
    if sh is not None:
        cap_y = cap_y + bf16_spacing(sh["ys"])
    out["y"] = np.minimum(b["y"], c * cap_y)
    if bwd is not None:
        cap_dx = bf16_spacing(bwd["dx"]) + (bf16_spacing(bwd["dxs"])[rows] * kept).sum(axis=1)
        if "dxs_s" in bwd:
            cap_dx = cap_dx + bf16_spacing(bwd["dxs_s"])
        out["dx"] = np.minimum(b["dx"], c * cap_dx)
    return out


# --------------------------------------------------------------------------
# some rows of one expert (sampled checks at full size)
# --------------------------------------------------------------------------

def expert_rows(xs, g, dy_rows, w_gate_e, w_up_e, w_down_e, store: str = "bf16") -> dict:
    """Every per-row quantity of some routed rows of one expert, from the
    layer's inputs: xs [R, H] the rows' tokens, g [R] their gates, dy_rows
    [R, H] (or None) the upstream gradients of their tokens.  The same steps
    and storage rounding points as ``forward`` and ``backward`` (SwiGLU
    expert of "MoE computation principle and execution process" section 2.3,
    its derivative, the combine backward's gate-weighted gather):
        G = xs.Wg, U = xs.Wu, A = silu(G) U, ys = A.Wd;
        dys = g dy, dA = dys.Wd^T, dG = dA U silu'(G), dU = dA silu(G),
        dxs = dG.Wg^T + dU.Wu^T.
    A row depends on its token and its expert alone, so any subset of a
    layer's rows gives the layer's values for those rows."""
    xs = as_f64(xs)
    wg, wu, wd = as_f64(w_gate_e), as_f64(w_up_e), as_f64(w_down_e)
    G, U, A, ys = swiglu_expert(xs, wg, wu, wd, store)
    out = dict(xs=xs, G=G, U=U, A=A, ys=ys)
    if dy_rows is None:
        return out
    dys = rho(as_f64(g).reshape(-1, 1) * as_f64(dy_rows), store)
    dA = dys @ wd.T
    sg = sigmoid(G)
    dG = rho(dA * U * sg * (1.0 + G * (1.0 - sg)), store)
    dU = rho(dA * (G * sg), store)
    dxs = rho(dG @ wg.T + dU @ wu.T, store)
    out.update(dys=dys, dG=dG, dU=dU, dxs=dxs)
    return out


# --------------------------------------------------------------------------
# slices of the expert weight gradients (sampled checks at full size)
# --------------------------------------------------------------------------

def weight_grad_slices(x, dy, topk, gates, e: int, w_gate_e, w_up_e, w_down_e, cols, store: str = "bf16") -> dict:
    """Columns ``cols`` of dW_gate[e] and dW_up[e] and rows ``cols`` of
    dW_down[e] from the layer's inputs and a given assignment (topk [N, K],
    gates [N, K]).

    The f-th column of G, U, A, dG and dU over expert e's rows is all these
    need, so the cost is a few matrix-vector products per column:
        rows   = the (n, k) with topk[n, k] == e;   xs = x[n], g = gates[n, k]
        G[:, f] = xs.Wg[:, f]   U[:, f] = xs.Wu[:, f]   A = silu(G) U
        dys    = g dy[n]        dA[:, f] = dys.Wd[f, :]
        dG     = dA U silu'(G)  dU = dA silu(G)
        dW_gate[:, f] = xs^T dG   dW_up[:, f] = xs^T dU   dW_down[f, :] = A^T dys
    with the same storage rounding points as ``forward`` / ``backward``.
    Returns dw_gate [H, C], dw_up [H, C], dw_down [C, H] (C = len(cols)).
    """
    x, dy = as_f64(x), as_f64(dy)
    topk = np.asarray(topk)
    N, K = topk.shape
    gflat = as_f64(gates).reshape(-1)
    flat = np.nonzero(topk.reshape(-1) == e)[0]
    tok = flat // K
    cols = np.asarray(cols, dtype=np.int64)
    wg = as_f64(w_gate_e)[:, cols]
    wu = as_f64(w_up_e)[:, cols]
    wd = as_f64(w_down_e)[cols, :]
    H = x.shape[1]
    xs = x[tok]
    dys = rho(gflat[flat][:, None] * dy[tok], store)
    G, U = rho(xs @ wg, store), rho(xs @ wu, store)
    A = rho(silu(G) * U, store)
    dA = dys @ wd.T
    sg = sigmoid(G)
    dG = rho(dA * U * sg * (1.0 + G * (1.0 - sg)), store)
    dU = rho(dA * (G * sg), store)
    out = dict(dw_gate=xs.T @ dG, dw_up=xs.T @ dU, dw_down=A.T @ dys)
    assert out["dw_gate"].shape == (H, cols.size)
    return out
