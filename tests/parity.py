"""Parity checks of a run of the layer (test infrastructure).

A run is judged at two levels.

Level 1 -- against the oracle, from the seeded inputs alone.  Every tensor the
run stores is compared with the oracle's value of the same tensor:
  * fp32 storage: max|err| <= 1e-4;
  * bf16 storage, bf16-stored tensors (xs, G, U, A, ys, y, dys, dG, dU, dxs,
    dx and the shared expert's): |err| <= 2e-2 + band per element, where the
    band (oracle.rounding_bands) is nonzero only where a rounding decision
    upstream was ambiguous and is capped at two bf16 spacings of the element
    (of the summed rows for y and dx); and rel-RMS <= 1e-2;
  * bf16 storage, float32 outputs (dgates, dlogits and the weight
    gradients): rel-RMS <= 1e-2; max|err| is reported.  These outputs are
    sums over H or over thousands of tokens of bf16-stored values, and two
    correct float32-accumulating runs that round some of those values to
    neighbouring bf16 numbers differ by more than 2e-2 (the float32
    evaluation in tests/test_parity_checker.py shows it), so an a-priori
    per-element bound against the oracle would be either loose or false.
    Level 2 holds them element by element instead.

Level 2 -- each step from the stored inputs of that step.  The step is
evaluated in float64 from the run's own stored inputs (x and the weights for
the first ones), and the run's output must be what float32 accumulation
gives: within the float32 summation bound (oracle.gemm_sigma and the
elementwise bounds below) for float32 outputs, and for bf16 outputs the
rounded value, or its neighbour only where the float64 value lies within
that bound of a rounding midpoint.  Because every step's inputs are checked
at Level 1 and every step's arithmetic at Level 2, a run that passes both is
a correct evaluation of the layer, and no dropped row, missing token, wrong
slot or transposed tile can hide in a loose band.

"Given the same assignment" the routing metadata is compared bit for bit.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from oracle import moe_oracle as O

U32 = 2.0 ** -24          # unit roundoff of float32
TOL_F32_ABS = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_RELRMS = 1e-2
BF16_STORED = ("xs", "G", "U", "A", "ys", "y", "dys", "dG", "dU", "dxs", "dx",
               "G_s", "U_s", "A_s", "ys_s", "dG_s", "dU_s", "dxs_s")
F32_OUTPUTS = ("dgates", "dlogits", "dw_r", "dw_gate", "dw_up", "dw_down", "dw_gate_s", "dw_up_s", "dw_down_s")


def _log(msg):
    print(msg, flush=True)


def rel_rms(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.mean(ref ** 2)) if ref.size else 0.0
    num = float(np.mean((got - ref) ** 2)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(np.sqrt(num / den))


# --------------------------------------------------------------------------
# access to a run's stored tensors
# --------------------------------------------------------------------------

class Run:
    """The stored tensors of a run (torch tensors on any device, or arrays),
    read as float64 or int64 on demand, whole or by rows and columns."""

    def __init__(self, **tensors):
        self.t = {k: v for k, v in tensors.items() if v is not None}

    def has(self, name: str) -> bool:
        return name in self.t

    def get(self, name: str, rows=None, cols=None) -> np.ndarray:
        v = self.t[name]
        if hasattr(v, "detach"):
            import torch
            if rows is not None:
                if isinstance(rows, slice):
                    v = v[rows]
                else:
                    v = v.index_select(0, torch.as_tensor(np.asarray(rows), dtype=torch.int64, device=v.device))
            if cols is not None:
                if isinstance(cols, slice):
                    v = v[:, cols]
                else:
                    v = v.index_select(1, torch.as_tensor(np.asarray(cols), dtype=torch.int64, device=v.device))
            return O.as_f64(v)
        a = np.asarray(v)
        if rows is not None:
            a = a[rows]
        if cols is not None:
            a = a[:, cols]
        return np.asarray(a, dtype=np.float64)

    def ints(self, name: str) -> np.ndarray:
        v = self.t[name]
        if hasattr(v, "detach"):
            v = v.detach().cpu().numpy()
        return np.asarray(v).astype(np.int64)


def weights_of(w_gate, w_up, w_down) -> Callable[[int], tuple]:
    """Expert e's (W_gate, W_up, W_down) in float64, converted on demand
    (one expert at a time, the last one cached)."""
    cache = {}

    def get(e: int):
        if e not in cache:
            cache.clear()
            cache[e] = (O.as_f64(w_gate[e]), O.as_f64(w_up[e]), O.as_f64(w_down[e]))
        return cache[e]
    return get


# --------------------------------------------------------------------------
# element checks
# --------------------------------------------------------------------------

def check_stored(name: str, got: np.ndarray, pre: np.ndarray, sigma: np.ndarray, store: str, log=_log) -> int:
    """Level 2 check of one step's stored output: `pre` is the step's exact
    value from its stored inputs and `sigma` bounds what float32
    accumulation may add to it.  bf16 storage: got is round(pre), or its
    neighbour where pre +- sigma reaches a rounding midpoint.  float32
    storage: |got - pre| <= sigma + 2 u |pre|.  Returns the number of
    elements on the other side of a midpoint (bf16)."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == pre.shape, (name, got.shape, pre.shape)
    if not np.all(np.isfinite(got)):
        raise AssertionError(f"{name}: non-finite values")
    if store == "bf16":
        rounded = O.round_bf16(pre)
        allowed = O.bf16_flip(pre, rounded, sigma)
        dev = np.abs(got - rounded)
    else:
        allowed = sigma + 2 * U32 * np.abs(pre)
        dev = np.abs(got - pre)
    bad = dev > allowed
    if bad.any():
        i = np.unravel_index(int(np.argmax(dev - allowed)), dev.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {dev.size} elements off the step's value; worst at "
                             f"{tuple(int(v) for v in i)}: got {got[i]:.6g}, step value {pre[i]:.6g}, "
                             f"allowed {allowed[i]:.3g}")
    flips = int(np.sum(dev > 0)) if store == "bf16" else 0
    log(f"[step] {name}: {dev.size} elements ok" + (f" ({flips} on the other side of a midpoint)" if flips else ""))
    return flips


def check_f32(name: str, got: np.ndarray, pre: np.ndarray, sigma: np.ndarray, log=_log):
    """Level 2 check of a float32 output: |got - pre| <= sigma."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == pre.shape, (name, got.shape, pre.shape)
    dev = np.abs(got - pre)
    bad = dev > sigma
    if bad.any() or not np.all(np.isfinite(got)):
        i = np.unravel_index(int(np.argmax(np.where(np.isfinite(dev), dev - sigma, np.inf))), dev.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {dev.size} elements off the step's value; worst at "
                             f"{tuple(int(v) for v in i)}: got {got[i]:.6g}, step value {pre[i]:.6g}, "
                             f"bound {sigma[i]:.3g}")
    log(f"[step] {name}: {dev.size} elements within the float32 bound (max|dev| {float(dev.max()) if dev.size else 0:.3e})")


def prod_sigma(a: np.ndarray, b: np.ndarray, store: str) -> np.ndarray:
    """float32 accumulation bound of a @ b; products of two bf16 values are
    exact in float32, products of float32 values add a rounding each."""
    s = O.gemm_sigma(a, b)
    if store != "bf16":
        s = s + 2 * U32 * (np.abs(a) @ np.abs(b))
    return s


def _silu_terms(G):
    s = O.sigmoid(G)
    d1 = s * (1.0 + G * (1.0 - s))
    # the device's sigmoid (hardware exponential of -g log2(e) and reciprocal)
    # carries a relative error of at most (4 + 2|g|) u; through 1 - s and the
    # product with g it adds an absolute error of s (1 + |g|)(8 + 4|g|) u to
    # the derivative d1, which matters where d1 itself is near zero
    es = (4.0 + 2.0 * np.abs(G)) * U32
    sig_d1 = s * (1.0 + np.abs(G)) * (8.0 + 4.0 * np.abs(G)) * U32 + 2 * es * np.abs(d1)
    return s, d1, es, sig_d1


# --------------------------------------------------------------------------
# Level 2: each step from its stored inputs
# --------------------------------------------------------------------------

def expert_of_rows(offsets: np.ndarray, rows: np.ndarray) -> np.ndarray:
    return np.searchsorted(offsets, rows, side="right") - 1


def check_metadata(run: Run, E: int, capacity: Optional[int], tile_m: int, log=_log):
    """Counts, bins, the stable sort, its inverse and the tile list of the
    run's own assignment: bit-exact."""
    topk = run.ints("topk")
    counts, offsets, sorted_flat, inv = O.routing_metadata(topk, E, capacity)
    for name, ref in (("counts", counts), ("offsets", offsets), ("sorted_flat", sorted_flat), ("inv", inv)):
        got = run.ints(name)
        if not np.array_equal(got, ref):
            bad = np.nonzero(got != ref)[0]
            raise AssertionError(f"{name}: {bad.size} entries differ, first at {int(bad[0])}")
    if run.has("tiles"):
        nt = int(run.ints("num_tiles").reshape(-1)[0])
        tl = O.tile_list(np.diff(offsets), offsets, tile_m)
        assert nt == len(tl), f"num_tiles {nt} != {len(tl)}"
        assert np.array_equal(run.ints("tiles")[:3 * nt].reshape(-1, 3), tl), "tile list"
    log(f"[step] metadata of {topk.size} routed rows bit-exact")


def check_rows_forward(x, weights, K: int, run: Run, rows, store: str, log=_log):
    """Permute, gate/up + SwiGLU and down on the given grouped rows."""
    off = run.ints("offsets")
    sf = run.ints("sorted_flat")
    rows = np.asarray(rows, dtype=np.int64)
    exp = expert_of_rows(off, rows)
    flips = 0
    for e in np.unique(exp):
        r = rows[exp == e]
        wg, wu, wd = weights(int(e))
        src = x[sf[r] // K]
        if run.has("xs"):
            xs = run.get("xs", rows=r)
            assert np.array_equal(xs, src), f"xs rows of expert {e} differ from x[sorted_flat / K]"
        G = run.get("G", rows=r) if run.has("G") else None
        U = run.get("U", rows=r) if run.has("U") else None
        A = run.get("A", rows=r)
        if G is not None:
            flips += check_stored(f"G (expert {e}, {r.size} rows)", G, src @ wg, prod_sigma(src, wg, store), store,
                                  log)
            flips += check_stored(f"U (expert {e}, {r.size} rows)", U, src @ wu, prod_sigma(src, wu, store), store,
                                  log)
            s, _, es, _ = _silu_terms(G)
            ap = G * s * U
            flips += check_stored(f"A (expert {e}, {r.size} rows)", A, ap, (es + 4 * U32) * np.abs(ap), store, log)
        else:
            # forward only: G and U are not stored; A is the rounding of silu
            # of the rounded G times the rounded U, so only its GEMM inputs
            # can be checked: recompute and allow the ambiguity of G and U
            Gp, Up = src @ wg, src @ wu
            Gr, Ur = O.rho(Gp, store), O.rho(Up, store)
            bG = O.bf16_flip(Gp, Gr, prod_sigma(src, wg, store)) if store == "bf16" else 0 * Gp
            bU = O.bf16_flip(Up, Ur, prod_sigma(src, wu, store)) if store == "bf16" else 0 * Up
            s, d1, es, _ = _silu_terms(Gr)
            ap = Gr * s * Ur
            sig = (es + 4 * U32) * np.abs(ap) + np.abs(Ur * d1) * bG + np.abs(Gr * s) * bU
            flips += check_stored(f"A (expert {e}, {r.size} rows, from x)", A, ap, sig, store, log)
        ys = run.get("ys", rows=r)
        flips += check_stored(f"ys (expert {e}, {r.size} rows)", ys, A @ wd, prod_sigma(A, wd, store), store, log)
    return flips


def check_rows_backward(weights, K: int, run: Run, dy, rows, store: str, log=_log):
    """Combine backward (dys), dA + SwiGLU backward and dX on the given
    grouped rows."""
    off = run.ints("offsets")
    sf = run.ints("sorted_flat")
    gflat = run.get("gates").reshape(-1)
    rows = np.asarray(rows, dtype=np.int64)
    exp = expert_of_rows(off, rows)
    for e in np.unique(exp):
        r = rows[exp == e]
        wg, wu, wd = weights(int(e))
        dysp = gflat[sf[r]][:, None] * dy[sf[r] // K]
        dys = run.get("dys", rows=r)
        check_stored(f"dys (expert {e}, {r.size} rows)", dys, dysp, 2 * U32 * np.abs(dysp), store, log)
        G, U = run.get("G", rows=r), run.get("U", rows=r)
        dA = dys @ wd.T
        sdA = prod_sigma(dys, wd.T, store)
        s, d1, es, sig_d1 = _silu_terms(G)
        dgp = dA * U * d1
        sdg = np.abs(U * d1) * sdA + np.abs(dA * U) * sig_d1 + 4 * U32 * np.abs(dgp)
        check_stored(f"dG (expert {e}, {r.size} rows)", run.get("dG", rows=r), dgp, sdg, store, log)
        dup = dA * G * s
        sdu = np.abs(G * s) * sdA + np.abs(dA * G * s) * es + 4 * U32 * np.abs(dup)
        check_stored(f"dU (expert {e}, {r.size} rows)", run.get("dU", rows=r), dup, sdu, store, log)
        dG, dU = run.get("dG", rows=r), run.get("dU", rows=r)
        dxp = dG @ wg.T + dU @ wu.T
        sdx = prod_sigma(dG, wg.T, store) + prod_sigma(dU, wu.T, store) + 2 * U32 * np.abs(dxp)
        check_stored(f"dxs (expert {e}, {r.size} rows)", run.get("dxs", rows=r), dxp, sdx, store, log)


def check_weight_grads(x, K: int, run: Run, store: str, experts=None, cols=None, log=_log):
    """dW_gate[e] = xs_e^T dG_e, dW_up[e] = xs_e^T dU_e, dW_down[e] = A_e^T dys_e
    (float32) for the given experts and columns of F (rows of dW_down);
    experts without rows: exact zeros."""
    off = run.ints("offsets")
    sf = run.ints("sorted_flat")
    E = off.size - 1
    experts = range(E) if experts is None else experts
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        c = slice(None) if cols is None else np.asarray(cols, dtype=np.int64)
        if r1 == r0:
            for name in ("dw_gate", "dw_up", "dw_down"):
                v = run.get(name, rows=[e])
                assert not v.any(), f"{name}[{e}] of an expert without rows is not zero"
            continue
        xs = x[sf[r0:r1] // K]
        dG = run.get("dG", rows=slice(r0, r1), cols=c)
        dU = run.get("dU", rows=slice(r0, r1), cols=c)
        A = run.get("A", rows=slice(r0, r1), cols=c)
        dys = run.get("dys", rows=slice(r0, r1))
        for name, a, b in (("dw_gate", xs.T, dG), ("dw_up", xs.T, dU), ("dw_down", A.T, dys)):
            pre = a @ b
            full = run.get(name, rows=[e])[0]
            got = full[:, c] if name != "dw_down" else full[c, :]
            check_f32(f"{name}[{e}] ({'all' if cols is None else len(cols)} columns, {r1 - r0} rows)", got, pre,
                      prod_sigma(a, b, store) + 2 * U32 * np.abs(pre), log)


def _token_chunks(N, size=2048, row_elems=0):
    """Token ranges of at most `size` tokens, fewer when each token gathers
    `row_elems` values (about 2^27 float64 values per range)."""
    if row_elems:
        size = max(64, min(size, (1 << 27) // row_elems))
    for n0 in range(0, N, size):
        yield slice(n0, min(N, n0 + size))


def check_combine(K: int, run: Run, store: str, shared: bool = False, log=_log):
    """y[n] = sum_k g[n,k] ys[inv[n,k]] (+ ys_s[n]), every token."""
    inv = run.ints("inv")
    g = run.get("gates")
    N = g.shape[0]
    flips = 0
    for t in _token_chunks(N, row_elems=K * run.t["ys"].shape[1]):
        iv = inv.reshape(N, K)[t]
        kept = iv >= 0
        ys = run.get("ys", rows=np.maximum(iv, 0).reshape(-1)).reshape(iv.shape[0], K, -1) * kept[:, :, None]
        terms = g[t][:, :, None] * ys
        pre = terms.sum(axis=1)
        sig = 4 * U32 * np.abs(terms).sum(axis=1)
        if shared:
            ys_s = run.get("ys_s", rows=t)
            pre = pre + ys_s
            sig = sig + 4 * U32 * np.abs(ys_s)
        flips += check_stored(f"y (tokens {t.start}..{t.stop - 1})", run.get("y", rows=t), pre, sig + 2 * U32 *
                              np.abs(pre), store, log=lambda m: None)
    log(f"[step] y: {N} tokens ok ({flips} elements on the other side of a midpoint)")


def check_combine_bwd_gates(K: int, run: Run, dy, log=_log):
    """dgates[n,k] = <dy[n], ys[inv[n,k]]> (float32; 0 for a dropped slot)."""
    inv = run.ints("inv")
    dg = run.get("dgates")
    N = dg.shape[0]
    H = dy.shape[1]
    worst = 0.0
    for t in _token_chunks(N, row_elems=K * H):
        iv = inv.reshape(N, K)[t]
        kept = iv >= 0
        ys = run.get("ys", rows=np.maximum(iv, 0).reshape(-1)).reshape(iv.shape[0], K, -1) * kept[:, :, None]
        prods = dy[t][:, None, :] * ys
        pre = prods.sum(axis=2)
        sig = 4 * U32 * np.sqrt(H) * np.sqrt((prods * prods).sum(axis=2)) + 6 * U32 * np.abs(pre)
        check_f32(f"dgates (tokens {t.start}..{t.stop - 1})", dg[t], pre, sig, log=lambda m: None)
        worst = max(worst, float(np.abs(dg[t] - pre).max()))
    log(f"[step] dgates: {N * K} entries within the float32 bound (max|dev| {worst:.3e})")


def check_route_bwd(x, K: int, run: Run, store: str, aux: Optional[dict] = None, log=_log):
    """dlogits from the stored gates and dgates (softmax over the selected
    logits, zero elsewhere; plus the balance-loss term when `aux` gives
    scale and the stored probabilities), and dW_r = x^T dlogits."""
    topk = run.ints("topk")
    g = run.get("gates")
    dg = run.get("dgates")
    dl = run.get("dlogits")
    N, E = dl.shape
    s = np.sum(g * dg, axis=1, keepdims=True)
    sel = g * (dg - s)
    pre = np.zeros((N, E))
    np.put_along_axis(pre, topk, sel, axis=1)
    sab = np.sum(np.abs(g * dg), axis=1, keepdims=True)
    sig_sel = 8 * U32 * (np.abs(sel) + g * sab)
    sig = np.zeros((N, E))
    np.put_along_axis(sig, topk, sig_sel, axis=1)
    if aux is not None:
        p = aux["probs"]
        f = aux["counts"].astype(np.float64) / (N * K)
        c = aux["scale"] * E / N
        sp = p @ f
        term = c * p * (f[None, :] - sp[:, None])
        pre = pre + term
        sig = sig + 16 * U32 * (np.abs(term) + abs(c) * p * (f[None, :] + sp[:, None])) + 4 * U32 * np.abs(pre)
    else:
        unsel = np.ones((N, E), dtype=bool)
        np.put_along_axis(unsel, topk, False, axis=1)
        assert not dl[unsel].any(), "unselected router logits must get exactly zero gradient"
    check_f32("dlogits", dl, pre, sig, log)
    ref = x.T @ dl
    check_f32("dW_r = x^T dlogits", run.get("dw_r"), ref, prod_sigma(x.T, dl, store) + 2 * U32 * np.abs(ref), log)


def check_permute_bwd(w_r, K: int, run: Run, store: str, shared: bool = False, log=_log):
    """dx[n] = sum_k dxs[inv[n,k]] + dlogits[n] W_r^T (+ dx_s[n]), every token."""
    inv = run.ints("inv")
    dl = run.get("dlogits")
    N = dl.shape[0]
    flips = 0
    for t in _token_chunks(N, row_elems=K * w_r.shape[0]):
        iv = inv.reshape(N, K)[t]
        kept = iv >= 0
        rows = run.get("dxs", rows=np.maximum(iv, 0).reshape(-1)).reshape(iv.shape[0], K, -1) * kept[:, :, None]
        d = dl[t]
        pre = rows.sum(axis=1) + d @ w_r.T
        sig = (4 * U32 * (np.abs(rows).sum(axis=1) + np.abs(d) @ np.abs(w_r.T)) + prod_sigma(d, w_r.T, store)
               + 2 * U32 * np.abs(pre))
        if shared:
            dxs_s = run.get("dxs_s", rows=t)
            pre = pre + dxs_s
            sig = sig + 4 * U32 * np.abs(dxs_s)
        flips += check_stored(f"dx (tokens {t.start}..{t.stop - 1})", run.get("dx", rows=t), pre, sig, store,
                              log=lambda m: None)
    log(f"[step] dx: {N} tokens ok ({flips} elements on the other side of a midpoint)")


def check_shared(x, shared_w, run: Run, store: str, dy=None, log=_log):
    """The shared expert's steps over every token (weight 1, rows = x)."""
    wg, wu, wd = (O.as_f64(w) for w in shared_w)
    G, U, A = run.get("G_s"), run.get("U_s"), run.get("A_s")
    check_stored("G_s", G, x @ wg, prod_sigma(x, wg, store), store, log)
    check_stored("U_s", U, x @ wu, prod_sigma(x, wu, store), store, log)
    s, d1, es, sig_d1 = _silu_terms(G)
    ap = G * s * U
    check_stored("A_s", A, ap, (es + 4 * U32) * np.abs(ap), store, log)
    check_stored("ys_s", run.get("ys_s"), A @ wd, prod_sigma(A, wd, store), store, log)
    if dy is None:
        return
    dA = dy @ wd.T
    sdA = prod_sigma(dy, wd.T, store)
    dgp = dA * U * d1
    check_stored("dG_s", run.get("dG_s"), dgp, np.abs(U * d1) * sdA + np.abs(dA * U) * sig_d1 + 4 * U32 * np.abs(dgp),
                 store, log)
    dup = dA * G * s
    check_stored("dU_s", run.get("dU_s"), dup, np.abs(G * s) * sdA + np.abs(dup) * es + 4 * U32 * np.abs(dup), store,
                 log)
    dG, dU = run.get("dG_s"), run.get("dU_s")
    dxp = dG @ wg.T + dU @ wu.T
    check_stored("dxs_s", run.get("dxs_s"), dxp, prod_sigma(dG, wg.T, store) + prod_sigma(dU, wu.T, store)
                 + 2 * U32 * np.abs(dxp), store, log)
    for name, a, b in (("dw_gate_s", x.T, dG), ("dw_up_s", x.T, dU), ("dw_down_s", A.T, dy)):
        pre = a @ b
        check_f32(name, run.get(name), pre, prod_sigma(a, b, store) + 2 * U32 * np.abs(pre), log)


def check_steps(x, w_r, weights, K: int, run: Run, store: str, dy=None, capacity=None, rows=None, dw_experts=None,
                dw_cols=None, shared_w=None, aux=None, tile_m: int = 256, log=_log):
    """Every step of a run from its own stored inputs (Level 2).

    x [N,H], w_r [H,E], dy [N,H] float64 host arrays; weights(e) gives
    expert e's float64 weights.  rows: grouped rows for the per-row GEMM
    steps (None: every kept row); dw_experts / dw_cols: experts and columns
    of F for the weight gradients (None: all)."""
    E = w_r.shape[1]
    check_metadata(run, E, capacity, tile_m, log)
    nkept = int(run.ints("offsets")[-1])
    rows = np.arange(nkept) if rows is None else np.asarray(rows, dtype=np.int64)
    check_rows_forward(x, weights, K, run, rows, store, log)
    if shared_w is not None:
        check_shared(x, shared_w, run, store, dy, log)
    check_combine(K, run, store, shared=shared_w is not None, log=log)
    if dy is None:
        return
    check_rows_backward(weights, K, run, dy, rows, store, log)
    check_combine_bwd_gates(K, run, dy, log)
    check_route_bwd(x, K, run, store, aux, log)
    check_weight_grads(x, K, run, store, dw_experts, dw_cols, log)
    check_permute_bwd(w_r, K, run, store, shared=shared_w is not None, log=log)


# --------------------------------------------------------------------------
# Level 1: against the oracle
# --------------------------------------------------------------------------

def compare_with_oracle(name: str, got, ref: np.ndarray, store: str, band=None, log=_log) -> dict:
    """One tensor against the oracle's (see the module docstring); returns
    max|err|, rel-RMS and the share of elements above 2e-2."""
    g = O.as_f64(got) if hasattr(got, "detach") else np.asarray(got, dtype=np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = np.abs(g - ref)
    emax = float(err.max()) if g.size else 0.0
    if store != "bf16":
        log(f"[oracle] {name}: max|err| {emax:.3e}")
        assert emax <= TOL_F32_ABS, f"{name}: max|err| {emax:.3e} > {TOL_F32_ABS:.0e}"
        return {"max_err": emax}
    rr = rel_rms(g, ref)
    over = float(np.mean(err > TOL_BF16_ABS)) if g.size else 0.0
    base = name.split("[")[0].split(" ")[0]
    if base in BF16_STORED:
        b = np.zeros_like(ref) if band is None else band
        excess = err - (TOL_BF16_ABS + b)
        worst = int(np.argmax(excess)) if g.size else 0
        msg = (f"[oracle] {name}: max|err| {emax:.3e}, rel-RMS {rr:.3e}; worst excess over 2e-2 + band "
               f"{excess.reshape(-1)[worst] if g.size else 0:.3e} at flat {worst}")
        log(msg)
        assert np.all(excess <= 0), msg
    else:
        log(f"[oracle] {name}: max|err| {emax:.3e} ({over:.2%} of elements above 2e-2), rel-RMS {rr:.3e}")
    assert rr <= TOL_BF16_RELRMS, f"{name}: rel-RMS {rr:.3e} > {TOL_BF16_RELRMS:.0e}"
    return {"max_err": emax, "rel_rms": rr, "frac_above_2e-2": over}
