"""A second implementation of the layer, for testing the parity checks on
the CPU: torch float32 on the CPU (its own summation order) with bf16
storage at the same points as the device path, given the oracle's routing.

It stands in for a device run: the parity checks must accept it, and must
reject it once a mistake is planted in any of its outputs.  It is test
infrastructure only and is never compared with the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch


def _f(a):
    return torch.tensor(np.asarray(a), dtype=torch.float32)


def _round_bf16(t):
    return t.to(torch.bfloat16).to(torch.float32)


def float32_layer(inp: dict, fwd: dict, K: int, backward: bool = True, store: str = "bf16") -> dict:
    """Forward (and backward) in float32 at the oracle's rounding points, given
    the oracle's assignment and metadata (fwd from oracle.forward).  Returns
    float64 arrays of every stored tensor plus the routing tensors.  store
    "f32" keeps every stored tensor in float32 (no bf16 rounding)."""
    rb = _round_bf16 if store == "bf16" else (lambda t: t)
    x, w_r = _f(inp["x"]), _f(inp["w_r"])
    wg, wu, wd = _f(inp["w_gate"]), _f(inp["w_up"]), _f(inp["w_down"])
    N, H = x.shape
    E = w_r.shape[1]
    sf = torch.tensor(fwd["sorted_flat"], dtype=torch.int64)
    inv = torch.tensor(fwd["inv"], dtype=torch.int64).view(N, K)
    off = [int(v) for v in fwd["offsets"]]
    gates = _f(fwd["gates"])
    tok = sf.clamp(min=0) // K
    NK, F = N * K, wg.shape[2]
    xs = torch.zeros(NK, H)
    xs[:off[E]] = x[tok[:off[E]]]
    G, U, A, ys = (torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, H))
    for e in range(E):
        s = slice(off[e], off[e + 1])
        G[s] = rb(xs[s] @ wg[e])
        U[s] = rb(xs[s] @ wu[e])
        A[s] = rb(torch.nn.functional.silu(G[s]) * U[s])
        ys[s] = rb(A[s] @ wd[e])
    kept = (inv >= 0).to(torch.float32)
    y = rb(sum(gates[:, k:k + 1] * kept[:, k:k + 1] * ys[inv[:, k].clamp(min=0)] for k in range(K)))
    out = dict(x=x, xs=xs, G=G, U=U, A=A, ys=ys, y=y)
    if backward:
        dy = _f(inp["dy"])
        grow = gates.reshape(-1)[sf.clamp(min=0)][:, None] * (sf >= 0).to(torch.float32)[:, None]
        dys = rb(grow * dy[tok])
        dgates = torch.stack([(dy * ys[inv[:, k].clamp(min=0)]).sum(1) * kept[:, k] for k in range(K)], 1)
        dG, dU, dxs = torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, H)
        dwg, dwu, dwd = torch.zeros_like(wg), torch.zeros_like(wu), torch.zeros_like(wd)
        for e in range(E):
            s = slice(off[e], off[e + 1])
            dA = dys[s] @ wd[e].T
            sg = torch.sigmoid(G[s])
            dG[s] = rb(dA * U[s] * sg * (1 + G[s] * (1 - sg)))
            dU[s] = rb(dA * G[s] * sg)
            dxs[s] = rb(dG[s] @ wg[e].T + dU[s] @ wu[e].T)
            dwg[e] = xs[s].T @ dG[s]
            dwu[e] = xs[s].T @ dU[s]
            dwd[e] = A[s].T @ dys[s]
        dl_sel = gates * (dgates - (gates * dgates).sum(1, keepdim=True))
        dlogits = torch.zeros(N, E).scatter_(1, torch.tensor(fwd["topk"], dtype=torch.int64), dl_sel)
        dw_r = x.T @ dlogits
        dx = rb(sum(dxs[inv[:, k].clamp(min=0)] * kept[:, k:k + 1] for k in range(K)) + dlogits @ w_r.T)
        out.update(dys=dys, dgates=dgates, dG=dG, dU=dU, dxs=dxs, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                   dlogits=dlogits, dw_r=dw_r, dx=dx)
    res = {k: v.double().numpy() for k, v in out.items() if k != "x"}
    for k in ("topk", "sorted_flat", "inv", "counts", "offsets"):
        res[k] = np.asarray(fwd[k]).astype(np.int64)
    res["gates"] = np.asarray(fwd["gates"], dtype=np.float64)
    return res
