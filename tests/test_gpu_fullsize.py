"""Parity at the full workload sizes, in the launch configuration the
benchmark times (MoELayerRunner: the same entry points, dims and stream).

The default workload (N=16384, H=512, F=1024, E=8, K=2) is compared element
by element with the whole-layer oracle, and every step of it from its own
stored inputs (tests/parity.py, both levels).  The larger workloads are
compared on what the oracle can compute one by one, so that every tile of
every grouped GEMM is in some oracle comparison:
  * the routing of every token: top-K bit-exact away from near-ties, gates;
  * the routing metadata and tile list of every row, bit-exact;
  * one row of every 256-row list tile of every expert (the last row of each
    expert's last, ragged tile): xs, G, U, A, ys (and dys, dG, dU, dxs)
    against the oracle's values of that row (oracle.expert_rows), within
    2e-2 plus two bf16 spacings, and each of those steps from the row's own
    stored inputs (tight);
  * sampled tokens (the first and last row of the hottest expert, the last
    row of a ragged tile, random ones): y, dgates, dlogits and dx against the
    oracle run on those tokens alone with the same assignment;
  * the weight gradients of every expert at one column of F in every
    256-wide block, over all H (so every 256 x 256 output tile): against the
    oracle (oracle.weight_grad_slices, rel-RMS) and from the run's own stored
    rows (tight); exact zeros for experts without rows;
  * the steps that are cheap at any size over every element: y = sum_k g
    ys[inv], dgates = <dy, ys[inv]>, dlogits, dW_r = x^T dlogits and
    dx = sum_k dxs[inv] + dlogits W_r^T.
"""
import numpy as np
import pytest
import torch

from moe_workloads import BASE, LARGE, SKEWED, WIDE, make_inputs
from oracle import moe_oracle as O
from tests import parity as P
from tests.gpu_common import (assert_close, assignment_mismatch, check_runner_steps, gpu_inputs, oracle_fwd,
                              runner_run, sync, to_np)

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
    _log("[full] every step from its stored inputs")
    check_runner_steps(cfg, cpu, r, y, grads)


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


def _tile_rows(tiles, seed=5):
    """One grouped row per list tile: a random row of each full tile, the
    last row of each expert's last tile."""
    rng = np.random.default_rng(seed)
    rows = []
    for i, (e, r0, n) in enumerate(tiles):
        last = i + 1 == len(tiles) or tiles[i + 1][0] != e
        rows.append(int(r0 + n - 1) if last else int(r0 + rng.integers(n)))
    return np.asarray(rows, dtype=np.int64)


def _rows(t, idx):
    return to_np(t[torch.as_tensor(idx, dtype=torch.int64, device=t.device)].cpu())


def _expert_w(dev, e):
    return tuple(to_np(dev[k][e].cpu()) for k in ("w_gate", "w_up", "w_down"))


def _tile_row_checks(cfg, dev, r, x, gates, rows):
    """Both levels on one row of every list tile: the oracle's values of the
    rows (from x and the weights alone) and each step from the rows' stored
    inputs."""
    K = cfg.K
    off = r.offsets.cpu().numpy().astype(np.int64)
    sf = r.sorted_flat.cpu().numpy().astype(np.int64)
    exp = P.expert_of_rows(off, rows)
    bufs = {"xs": r.xs, "G": r.g, "U": r.u, "A": r.act, "ys": r.ys}
    run = runner_run(r)
    dy = None
    if cfg.backward:
        bufs.update({"dys": r.dys, "dG": r.dg, "dU": r.du, "dxs": r.dxs})
        run.t.update(dys=r.dys, dG=r.dg, dU=r.du, dxs=r.dxs)
        dy = _host(dev["dy"])
    quiet = lambda msg: None  # noqa: E731
    worst = {}
    for e in np.unique(exp):
        rr = rows[exp == e]
        tok = sf[rr] // K
        w = _expert_w(dev, int(e))
        ref = O.expert_rows(x[tok], gates.reshape(-1)[sf[rr]], None if dy is None else dy[tok], *w, "bf16")
        for name, buf in bufs.items():
            if buf is None:
                continue
            band = O.BAND_CAP_SPACINGS * O.bf16_spacing(ref[name])
            m = P.compare_with_oracle(f"{name}[expert {e}, {rr.size} tile rows]", _rows(buf, rr), ref[name], "bf16",
                                      band=band, log=quiet)
            worst[name] = max(worst.get(name, 0.0), m["max_err"])
        # each step of those rows from its own stored inputs
        P.check_rows_forward(x, lambda _e: w, K, run, rr, "bf16", log=quiet)
        if dy is not None:
            P.check_rows_backward(lambda _e: w, K, run, dy, rr, "bf16", log=quiet)
    for name, v in worst.items():
        _log(f"[tile rows] {name}: {rows.size} rows (one per list tile) vs the oracle, max|err| {v:.3e}")
    _log(f"[tile rows] every step of the {rows.size} rows from its stored inputs")


def _sampled_token_checks(cfg, dev, r, x, topk, gates, tokens, y, grads):
    """The oracle on the sampled tokens alone, same assignment, experts
    restricted to the ones they use: the token-level outputs y, dgates,
    dlogits and dx."""
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
    if cfg.backward:
        dy_s = _rows(dev["dy"], tsel)
        ob = O.backward(of, dy_s)
        bd = O.rounding_bands(of, ob, dy_s)
    else:
        bd = O.rounding_bands(of)
    assert_close("y[sampled]", _rows(y, tsel), of["y"], "bf16", band=bd["y"])
    if cfg.backward:
        assert_close("dgates[sampled]", _rows(grads["dgates"], tsel), ob["dgates"], "bf16")
        dl = _rows(grads["dlogits"], tsel)
        assert_close("dlogits[sampled]", dl[:, used], ob["dlogits"], "bf16")
        others = np.setdiff1d(np.arange(cfg.E), used)
        assert not dl[:, others].any(), "unselected logits must get exactly zero gradient"
        assert_close("dx[sampled]", _rows(grads["dx"], tsel), ob["dx"], "bf16", band=bd["dx"])


def _weight_grad_checks(cfg, dev, r, x, topk, gates, counts, grads):
    """Every expert's weight gradients at one column of F per 256-wide block
    (all H): against the oracle's slices, and from the run's stored rows."""
    dy = _host(dev["dy"])
    rng = np.random.default_rng(3)
    cols = np.asarray([b + int(rng.integers(min(256, cfg.F - b))) for b in range(0, cfg.F, 256)], dtype=np.int64)
    c = torch.as_tensor(cols, dtype=torch.int64, device=DEV)
    worst = {}
    for e in np.where(counts > 0)[0]:
        e = int(e)
        wg, wu, wd = _expert_w(dev, e)
        s = O.weight_grad_slices(x, dy, topk, gates, e, wg, wu, wd, cols, "bf16")
        for name, got in (("dw_gate", grads["dw_gate"][e].index_select(1, c)),
                          ("dw_up", grads["dw_up"][e].index_select(1, c)),
                          ("dw_down", grads["dw_down"][e].index_select(0, c))):
            m = P.compare_with_oracle(f"{name}[{e}][{cols.size} columns]", to_np(got.cpu()), s[name], "bf16",
                                      log=lambda msg: None)
            worst[name] = max(worst.get(name, 0.0), m["max_err"])
    for name, v in worst.items():
        _log(f"[dW] {name}: {int((counts > 0).sum())} experts x {cols.size} columns (one per 256-block) vs the "
             f"oracle, max|err| {v:.3e}")
    run = runner_run(r, None, grads)
    P.check_weight_grads(x, cfg.K, run, "bf16", experts=range(cfg.E), cols=cols, log=lambda msg: None)
    _log(f"[dW] every expert's weight gradients at {cols.size} columns per matrix: every element from the stored "
         f"rows; experts without rows exactly zero")


def _whole_tensor_steps(cfg, dev, r, x, grads, y):
    """The steps that are cheap at any size, over every element."""
    run = runner_run(r, y, grads)
    P.check_combine(cfg.K, run, "bf16")
    if not cfg.backward:
        return
    P.check_combine_bwd_gates(cfg.K, run, _host(dev["dy"]))
    P.check_route_bwd(x, cfg.K, run, "bf16")
    P.check_permute_bwd(_host(dev["w_r"]), cfg.K, run, "bf16")


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
    from mixture_experts_layer_sort_amd import _lib as L
    rows = _tile_rows(O.tile_list(counts, offsets, L.MOE_TILE_M))
    _tile_row_checks(cfg, dev, r, x, gates, rows)
    tokens = _sample_tokens(cfg, counts, offsets, sorted_flat, n_random)
    _sampled_token_checks(cfg, dev, r, x, topk, gates, tokens, y, grads)
    if cfg.backward:
        _weight_grad_checks(cfg, dev, r, x, topk, gates, counts, grads)
    _whole_tensor_steps(cfg, dev, r, x, grads, y)
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
