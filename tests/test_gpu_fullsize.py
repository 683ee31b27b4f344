"""Parity at the full workload sizes, in the launch configuration the
benchmark times (MoELayerRunner: the same entry points, dims and stream).

The default workload (N=16384, H=512, F=1024, E=8, K=2) is compared element
by element with the whole-layer oracle.  The larger workloads are compared on
what the oracle can compute one by one:
  * the routing of every token: top-K bit-exact away from near-ties, gates;
  * the routing metadata and tile list of every row, bit-exact;
  * sampled tokens (the first and last row of the hottest expert, the last
    row of a ragged tile, random ones): every stored intermediate of their K
    rows, y, dgates, dlogits and dx, against the oracle run on those tokens
    alone with the same assignment (experts restricted to the ones they
    use), with rounding bands;
  * sampled columns of dW_gate / dW_up and rows of dW_down of the hottest, a
    middle and the coldest non-empty expert, with bands; exact zeros for
    experts without rows;
  * properties that hold at any size, over every element: y = sum_k g ys[inv],
    dx = sum_k dxs[inv] + dlogits W_r^T, dW_r = x^T dlogits, and
    dW_gate[e] = xs_e^T dG_e on a column slice of the hottest expert.
"""
import numpy as np
import pytest
import torch

from moe_workloads import BASE, LARGE, SKEWED, WIDE, make_inputs
from oracle import moe_oracle as O
from tests.gpu_common import assert_close, assignment_mismatch, gpu_inputs, oracle_fwd, sync, to_np

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()  # fails loudly when the HIP library is missing
    yield
    torch.cuda.empty_cache()


def _runner(cfg):
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    return MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", backward=cfg.backward)


def _log(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------
# default workload: every element against the whole-layer oracle
# --------------------------------------------------------------------------

def test_default_workload_every_element():
    cfg = BASE
    _log(f"[full] {cfg.name}: inputs")
    cpu, dev = gpu_inputs(cfg, 0, with_dy=True)
    r = _runner(cfg)
    r.route(dev["x"], dev["w_r"], dev["bias"])
    sync()
    _log("[full] oracle forward")
    of = oracle_fwd(cfg, cpu)
    bad = assignment_mismatch(r.topk.cpu().numpy(), of, cfg.K)
    assert len(bad) <= max(1, cfg.N // 1000)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"],
                  topk=torch.from_numpy(of["topk"]).cuda(),
                  gates=torch.from_numpy(of["gates"].astype(np.float32)).cuda())
    grads = r.backward(dev["dy"])
    sync()
    _log("[full] oracle backward and bands")
    ob = O.backward(of, cpu["dy"])
    bd = O.rounding_bands(of, ob, cpu["dy"])
    ref = dict(of)
    ref.update(ob)
    got = {"xs": r.xs, "G": r.g, "U": r.u, "A": r.act, "ys": r.ys, "y": y, "dys": r.dys,
           "dgates": grads["dgates"], "dlogits": grads["dlogits"], "dG": r.dg, "dU": r.du, "dxs": r.dxs,
           "dx": grads["dx"], "dw_r": grads["dw_r"], "dw_gate": grads["dw_gate"], "dw_up": grads["dw_up"],
           "dw_down": grads["dw_down"]}
    for name, t in got.items():
        if t is not None:                 # xs: gathered from x, never materialised
            assert_close(name, t, ref[name], "bf16", band=bd.get(name))
    nt = int(r.num_tiles.item())
    from mixture_experts_layer_sort_amd import _lib as L
    assert np.array_equal(r.tiles.cpu().numpy()[:3 * nt].reshape(-1, 3),
                          O.tile_list(of["counts"], of["offsets"], L.MOE_TILE_M))


# --------------------------------------------------------------------------
# larger workloads: sampled outputs and properties
# --------------------------------------------------------------------------

def _host(t):
    return None if t is None else to_np(t.cpu())


def _route_all_tokens(cfg, dev, r):
    """Oracle routing of every token from float64 logits; checks the GPU's."""
    x, w_r, bias = _host(dev["x"]), _host(dev["w_r"]), _host(dev["bias"])
    logits = O.router_logits(x, w_r, bias)
    topk = O.topk_experts(logits, cfg.K)
    gates = O.rho32(O.gates_topk_softmax(logits, topk), "bf16")
    r.route(dev["x"], dev["w_r"], dev["bias"])
    sync()
    bad = assignment_mismatch(r.topk.cpu().numpy(), {"topk": topk, "logits": logits}, cfg.K)
    assert len(bad) <= max(1, cfg.N // 1000), f"{len(bad)} tokens routed differently"
    good = np.setdiff1d(np.arange(cfg.N), bad)
    g = r.gates.cpu().numpy().astype(np.float64)
    # float32 logits are within gemm_sigma of the exact ones; a gate moves by
    # at most 2 g_k max_j |dl_j| under logit changes dl, plus a few float32
    # roundings of the softmax
    dl = np.take_along_axis(O.gemm_sigma(x, w_r), topk.astype(np.int64), axis=1).max(axis=1, keepdims=True)
    tol = 2.0 * gates * dl + 8 * U32
    worst = float(np.max(np.abs(g[good] - gates[good]) - tol[good]))
    _log(f"[sampled] gates: max|err| {float(np.max(np.abs(g[good] - gates[good]))):.3e}, worst err - bound {worst:.3e}")
    assert worst <= 0
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-6)
    _log(f"[sampled] routing of {cfg.N} tokens checked ({len(bad)} near-ties)")
    return x, logits, topk, gates


def _metadata_exact(cfg, r, topk):
    from mixture_experts_layer_sort_amd import _lib as L
    counts, offsets, sorted_flat, inv = O.routing_metadata(topk, cfg.E)
    assert np.array_equal(r.counts.cpu().numpy(), counts)
    assert np.array_equal(r.offsets.cpu().numpy(), offsets)
    assert np.array_equal(r.sorted_flat.cpu().numpy(), sorted_flat)
    assert np.array_equal(r.inv.cpu().numpy(), inv)
    nt = int(r.num_tiles.item())
    assert np.array_equal(r.tiles.cpu().numpy()[:3 * nt].reshape(-1, 3), O.tile_list(counts, offsets, L.MOE_TILE_M))
    _log(f"[sampled] metadata of {cfg.N * cfg.K} rows bit-exact, {nt} tiles")
    return counts, offsets, sorted_flat, inv


def _sample_tokens(cfg, counts, offsets, sorted_flat, n_random, seed=11):
    K = cfg.K
    hot = int(np.argmax(counts))
    picks = [int(sorted_flat[offsets[hot]]) // K, int(sorted_flat[offsets[hot + 1] - 1]) // K]
    ragged = [e for e in range(cfg.E) if counts[e] % 256 and e != hot]
    if ragged:
        e = ragged[len(ragged) // 2]
        picks.append(int(sorted_flat[offsets[e + 1] - 1]) // K)
    rng = np.random.default_rng(seed)
    picks += [int(v) for v in rng.choice(cfg.N, n_random, replace=False)]
    return sorted(set(picks))


def _rows(t, idx):
    return to_np(t[torch.as_tensor(idx, dtype=torch.int64, device=t.device)].cpu())


def _sampled_token_checks(cfg, dev, r, x, topk, gates, tokens, y, grads):
    """The oracle on the sampled tokens alone, same assignment, experts
    restricted to the ones they use."""
    K = cfg.K
    tsel = np.asarray(tokens)
    top_s = topk[tsel]
    used = np.unique(top_s)
    remap = np.full(cfg.E, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    idx = torch.as_tensor(used, dtype=torch.int64, device=DEV)
    _log(f"[sampled] {len(tokens)} tokens use {used.size} experts")
    wg = to_np(dev["w_gate"].index_select(0, idx).cpu())
    wu = to_np(dev["w_up"].index_select(0, idx).cpu())
    wd = to_np(dev["w_down"].index_select(0, idx).cpu())
    w_r = _host(dev["w_r"])
    bias = _host(dev["bias"])
    of = O.forward(x[tsel], w_r[:, used], wg, wu, wd, K, bias=None if bias is None else bias[used], store="bf16",
                   topk=remap[top_s])
    assert np.max(np.abs(of["gates"] - gates[tsel])) <= 1e-7
    ob = None
    if cfg.backward:
        dy_s = _rows(dev["dy"], tsel)
        ob = O.backward(of, dy_s)
        bd = O.rounding_bands(of, ob, dy_s)
    else:
        bd = O.rounding_bands(of)
    inv_gpu = r.inv.cpu().numpy().astype(np.int64)
    gpu_rows = inv_gpu.reshape(cfg.N, K)[tsel].reshape(-1)      # token-major (i, k)
    ora_rows = of["inv"].reshape(len(tokens), K).reshape(-1)
    # a forward-only runner gathers the rows inside gate/up and holds no xs
    names = (["xs"] if r.xs is not None else []) + ["G", "U", "A", "ys"] + (
        ["dys", "dG", "dU", "dxs"] if cfg.backward else [])
    bufs = {"xs": r.xs, "G": r.g, "U": r.u, "A": r.act, "ys": r.ys}
    if cfg.backward:
        bufs.update({"dys": r.dys, "dG": r.dg, "dU": r.du, "dxs": r.dxs})
    ref = dict(of)
    if ob is not None:
        ref.update(ob)
    for name in names:
        if bufs[name] is None:
            continue
        band = bd.get(name)
        assert_close(f"{name}[sampled rows]", _rows(bufs[name], gpu_rows), ref[name][ora_rows], "bf16",
                     band=None if band is None else band[ora_rows])
    assert_close("y[sampled]", _rows(y, tsel), of["y"], "bf16", band=bd["y"])
    if cfg.backward:
        assert_close("dgates[sampled]", _rows(grads["dgates"], tsel), ob["dgates"], "bf16", band=bd["dgates"])
        dl = _rows(grads["dlogits"], tsel)
        assert_close("dlogits[sampled]", dl[:, used], ob["dlogits"], "bf16", band=bd["dlogits"])
        others = np.setdiff1d(np.arange(cfg.E), used)
        assert not dl[:, others].any(), "unselected logits must get exactly zero gradient"
        assert_close("dx[sampled]", _rows(grads["dx"], tsel), ob["dx"], "bf16", band=bd["dx"])


def _weight_grad_checks(cfg, dev, r, x, topk, gates, counts, grads):
    dy = _host(dev["dy"])
    nonempty = np.where(counts > 0)[0]
    order = nonempty[np.argsort(counts[nonempty], kind="stable")]
    experts = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    rng = np.random.default_rng(3)
    cols = sorted({0, int(rng.integers(1, cfg.F - 1)), cfg.F - 1})
    for e in experts:
        s = O.weight_grad_slices(x, dy, topk, gates, e, to_np(dev["w_gate"][e].cpu()), to_np(dev["w_up"][e].cpu()),
                                 to_np(dev["w_down"][e].cpu()), cols, "bf16")
        c = torch.as_tensor(cols, dtype=torch.int64, device=DEV)
        assert_close(f"dw_gate[{e}][:, {cols}]", to_np(grads["dw_gate"][e].index_select(1, c).cpu()), s["dw_gate"],
                     "bf16", band=s["band_dw_gate"])
        assert_close(f"dw_up[{e}][:, {cols}]", to_np(grads["dw_up"][e].index_select(1, c).cpu()), s["dw_up"],
                     "bf16", band=s["band_dw_up"])
        assert_close(f"dw_down[{e}][{cols}, :]", to_np(grads["dw_down"][e].index_select(0, c).cpu()),
                     s["dw_down"], "bf16", band=s["band_dw_down"])
    for e in np.where(counts == 0)[0]:
        for name in ("dw_gate", "dw_up", "dw_down"):
            assert torch.count_nonzero(grads[name][int(e)]).item() == 0, f"{name}[{e}] of an empty expert"


def _within(name, got, pre, sigma):
    """|got - pre| <= sigma element by element (got float32 results)."""
    dev = np.abs(to_np(got) - pre)
    worst = float((dev - sigma).max())
    _log(f"{name}: max|dev| {float(dev.max()):.3e}, worst dev - bound {worst:.3e}")
    assert worst <= 0, name


def _rounded_within(name, got, pre, sigma):
    """A bf16 result of a float32 sum whose exact value is pre (to within
    sigma): equal to round(pre) unless the interval reaches a midpoint."""
    rounded = O.round_bf16(pre)
    band = O.bf16_flip(pre, rounded, sigma)
    dev = np.abs(to_np(got) - rounded)
    assert np.all(dev <= band), f"{name}: {int(np.sum(dev > band))} elements off"
    _log(f"{name}: {int(np.sum(dev > 0))} of {dev.size} elements on the other side of a midpoint, all within band")


def _property_checks(cfg, dev, r, x, grads, y):
    K = cfg.K
    inv = r.inv.cpu().numpy().astype(np.int64).reshape(cfg.N, K)
    g = r.gates.cpu().numpy().astype(np.float64)
    ys = to_np(r.ys.cpu())
    terms = g[:, :, None] * ys[inv]
    _rounded_within("y = sum_k g ys[inv]", y.cpu(), terms.sum(axis=1), 8 * U32 * np.abs(terms).sum(axis=1))
    del ys, terms
    if not cfg.backward:
        return
    dxs = to_np(r.dxs.cpu())
    dl = to_np(grads["dlogits"].cpu())
    w_r = _host(dev["w_r"])
    rows = dxs[inv].sum(axis=1)
    pre = rows + dl @ w_r.T
    sig = 8 * U32 * (np.abs(dxs[inv]).sum(axis=1) + np.abs(dl) @ np.abs(w_r.T)) + O.gemm_sigma(dl, w_r.T)
    _rounded_within("dx = sum_k dxs[inv] + dlogits W_r^T", grads["dx"].cpu(), pre, sig)
    del dxs, rows, pre, sig
    ref = x.T @ dl
    _within("dW_r = x^T dlogits", grads["dw_r"].cpu(), ref, O.gemm_sigma(x.T, dl) + 2 * U32 * np.abs(ref))
    counts = r.counts.cpu().numpy()
    off = r.offsets.cpu().numpy()
    e = int(np.argmax(counts))
    sl = slice(int(off[e]), int(off[e + 1]))
    cols = slice(cfg.F - 128, cfg.F)
    # the expert's rows of the grouped order, x[sorted_flat / K]
    src = r.sorted_flat[sl].long() // cfg.K
    xs_e = to_np(dev["x"][src].cpu())
    dG_e = to_np(r.dg[sl, cols].cpu())
    ref = xs_e.T @ dG_e
    _within(f"dW_gate[{e}] = xs_e^T dG_e (last 128 columns)", grads["dw_gate"][e][:, cols].cpu(), ref,
            O.gemm_sigma(xs_e.T, dG_e) + 2 * U32 * np.abs(ref))


@pytest.mark.parametrize("cfg,n_random", [(SKEWED, 2), (LARGE, 1), (WIDE, 0)], ids=lambda v: getattr(v, "name", ""))
def test_large_workload_sampled(cfg, n_random):
    _log(f"[sampled] {cfg.name}: inputs on the device")
    dev = make_inputs(cfg, 0, device=DEV, with_dy=cfg.backward)
    r = _runner(cfg)
    x, logits, topk, gates = _route_all_tokens(cfg, dev, r)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"],
                  topk=torch.from_numpy(topk).to(DEV), gates=torch.from_numpy(gates.astype(np.float32)).to(DEV))
    grads = r.backward(dev["dy"]) if cfg.backward else None
    sync()
    counts, offsets, sorted_flat, inv = _metadata_exact(cfg, r, topk)
    tokens = _sample_tokens(cfg, counts, offsets, sorted_flat, n_random)
    _sampled_token_checks(cfg, dev, r, x, topk, gates, tokens, y, grads)
    if cfg.backward:
        _weight_grad_checks(cfg, dev, r, x, topk, gates, counts, grads)
    _property_checks(cfg, dev, r, x, grads, y)
    del r, dev
    torch.cuda.empty_cache()


def test_large_ffn_bitwise_identical_across_three_runs():
    """Outputs and every gradient (dX, dW_gate/up/down, dW_r) byte-identical
    across three whole-layer runs, the second with poisoned buffers."""
    cfg = LARGE
    _log(f"[determinism] {cfg.name}")
    dev = make_inputs(cfg, 1, device="cuda", with_dy=True)
    r = _runner(cfg)
    first = None
    for rep in range(3):
        if rep == 1:
            for t in (r.y, r.dx, r.dw_gate, r.dw_up, r.dw_down, r.dw_r, r.xs, r.act, r.ys, r.dg, r.du):
                if t is not None:
                    t.fill_(float("nan"))
        y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
        grads = r.backward(dev["dy"])
        sync()
        outs = [y] + [grads[k] for k in ("dx", "dw_gate", "dw_up", "dw_down", "dw_r", "dgates", "dlogits")]
        outs = [o.clone() for o in outs]
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                bits = torch.int32 if a.dtype == torch.float32 else torch.int16
                assert torch.equal(a.view(bits), b.view(bits))
        _log(f"[determinism] run {rep} done")
    del r, dev, first
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [BASE, SKEWED, LARGE], ids=lambda c: c.name)
def test_gathered_weight_gradients_at_full_size(cfg):
    """The weight gradients reading x through sorted_flat (no xs, as
    bench.py --dw-gather runs them) give the same bytes as the default
    launch configuration, whose results the tests above check against the
    oracle."""
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    _log(f"[dw_gather] {cfg.name}")
    dev = make_inputs(cfg, 2, device=DEV, with_dy=True)
    outs = []
    for dwg in (False, True):
        r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, DEV, dw_gather=dwg)
        assert (r.xs is None) == dwg
        y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
        g = r.backward(dev["dy"])
        sync()
        outs.append([y.clone()] + [g[k].clone() for k in ("dx", "dw_gate", "dw_up", "dw_down", "dw_r")])
        del r, y, g
        torch.cuda.empty_cache()
    for name, a, b in zip(("y", "dx", "dw_gate", "dw_up", "dw_down", "dw_r"), outs[0], outs[1]):
        bits = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(bits), b.view(bits)), name
    del dev, outs
    torch.cuda.empty_cache()
