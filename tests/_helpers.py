"""Shared helpers of the GPU tests: upload generator inputs, run the library, run the oracle."""
from __future__ import annotations

import numpy as np

import datagen
from datagen import BF16, F32

TOL = {F32: 1e-5, BF16: 2e-3}


def to_device(x: np.ndarray, dev):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev)
    return torch.from_numpy(x).to(dev)


def host_inputs(w, first=0, n=None, layers=None):
    layers = range(w.n_layers) if layers is None else layers
    n = w.B if n is None else n
    As = [datagen.host_tensor(w, l, 0, first, n) for l in layers]
    Gs = [datagen.host_tensor(w, l, 1, first, n) for l in layers]
    return As, Gs


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return np.linalg.norm(got - want) / (den if den > 0 else 1.0)


def max_rel(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-300))) if want.size else 0.0


def gpu_step(w, As, Gs, dev, C=None, sigma=None, seed=0, step=0, flags=0, path=0, sum_policy=0,
             n_records=None, plan=None, ws=None, out=None):
    """Run dpsgd_step on uploaded copies of the host inputs.  Returns dict of numpy arrays."""
    import torch
    import differentially_private_amd as dp
    C = w.C if C is None else C
    sigma = w.sigma if sigma is None else sigma
    n = As[0].shape[0] if n_records is None else n_records
    if plan is None:
        plan = dp.Plan(w.layers, w.dtype, max(n, 1), w.T, path, sum_policy)
    dA = [to_device(a, dev) for a in As]
    dG = [to_device(g, dev) for g in Gs]
    if out is None:
        out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=dev)
               for a, b in w.layers]
    if ws is None:
        ws = plan.workspace(dev)
    nrm = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=dev)
    cf = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=dev)
    dp.step(plan, dA, dG, out, ws, C, sigma, seed, step, n_records=n, flags=flags, norms_out=nrm,
            clip_out=cf)
    st = dp.status(plan, ws)
    torch.cuda.synchronize()
    return {"n": nrm.cpu().numpy()[:n], "c": cf.cpu().numpy()[:n],
            "out": [o.cpu().numpy().reshape(a, b) for o, (a, b) in zip(out, w.layers)],
            "status": st, "plan": plan, "ws": ws, "dA": dA, "dG": dG, "out_dev": out}


def flat(xs):
    return np.concatenate([np.asarray(x, dtype=np.float64).reshape(-1) for x in xs])


def device_tensor(w, layer, tensor, first, n, dev):
    """Generator output for records [first, first+n) of (layer, tensor), filled directly in HBM."""
    import torch
    scale, heavy = datagen.record_params(w, layer, tensor, first, n)
    ds = torch.from_numpy(scale).to(dev)
    dh = torch.from_numpy(heavy).to(dev)
    d = datagen.tensor_dim(w, layer, tensor)
    buf = torch.empty((n, w.T, d), dtype=torch.float32 if w.dtype == F32 else torch.int16,
                      device=dev)
    datagen.device_fill(w, layer, tensor, buf.data_ptr(), first, n, ds.data_ptr(), dh.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    return buf


def oracle_record_layer_norm2(w, rec, layers):
    """Oracle squared norm of record `rec`'s gradient in each of `layers` (inputs regenerated)."""
    import oracle
    out = []
    for l in layers:
        A = datagen.host_tensor(w, l, 0, rec, 1)
        G = datagen.host_tensor(w, l, 1, rec, 1)
        out.append(oracle.layer_norm2(A, G)[0])
    return np.array(out)


def oracle_sum_entry(w, layer, j, k, c, first=0, n=None):
    """Oracle S_layer[j, k] = sum_i c_i sum_t A[i,t,j] G[i,t,k] over records [first, first+n),
    from gathered columns of the generator (the gradient entry of every record, weighted)."""
    import oracle
    n = w.B if n is None else n
    rec = np.repeat(np.arange(first, first + n), w.T)
    tok = np.tile(np.arange(w.T), n)
    a = datagen.gather(w, layer, 0, rec, tok, np.full(rec.size, j))
    g = datagen.gather(w, layer, 1, rec, tok, np.full(rec.size, k))
    S = oracle.layer_clipped_sum(a.reshape(n, w.T, 1), g.reshape(n, w.T, 1),
                                 np.asarray(c, dtype=np.float64))
    return S[0, 0]
