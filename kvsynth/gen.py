"""Seeded generators: AR(1) keys, Gaussian values and queries, outlier masks.

Every random stream is keyed by SeedSequence([workload id, batch, layer, kv_head, tag]),
so any subset of slices can be regenerated on its own.  Large caches are generated
with torch on the target device (fp32, then rounded to the storage type); tiny ones
for CPU tests with numpy.

Data recipe:
  keys   k_0 ~ N(0, I); k_t = rho * k_{t-1} + sigma * eps_t, eps_t ~ N(0, I); sigma
         defaults to sqrt(1 - rho^2) (unit stationary variance); rho is fixed or drawn
         uniformly per (layer, kv head); an optional per-(layer, kv head) mean vector
         mu ~ N(0, mean_std^2 I) is added to every key.  Appended decode keys continue
         each slice's AR(1) sequence.
  values iid N(0, 1); queries iid N(0, 1) per (group, q head, step).
  outlier mask: round(frac * layers * H_kv) (layer, kv head) pairs drawn without
         replacement, the same pairs for every batch element.
"""

import math

import numpy as np

TAGS = {"K": 1, "V": 2, "q": 3, "mu": 4, "rho": 5, "mask": 6, "app_v": 7}


def seed_of(cid, batch, layer, head, tag):
    ss = np.random.SeedSequence([int(cid), int(batch), int(layer), int(head), TAGS[tag]])
    return int(ss.generate_state(1, np.uint32)[0])


def _slice_coords(w, z):
    group, head = divmod(z, w.H_kv)
    b, layer = divmod(group, w.layers)
    return b, layer, head


def slice_params(w, z):
    """(rho, sigma, mu or None) of slice z."""
    _, layer, head = _slice_coords(w, z)
    lo, hi = w.rho
    if lo == hi:
        rho = float(lo)
    else:
        rho = float(np.random.default_rng(seed_of(w.cid, 0, layer, head, "rho")).uniform(lo, hi))
    sigma = w.sigma if w.sigma is not None else math.sqrt(1.0 - rho * rho)
    mu = None
    if w.mean_std > 0:
        mu = np.random.default_rng(seed_of(w.cid, 0, layer, head, "mu")).normal(
            0.0, w.mean_std, size=w.d)
    return rho, sigma, mu


def outlier_mask(w):
    """uint8 [slices]: 1 for slices whose (layer, kv head) is flagged outlier."""
    mask = np.zeros(w.slices, dtype=np.uint8)
    count = int(round(w.outlier_frac * w.layers * w.H_kv))
    if count == 0:
        return mask
    rng = np.random.default_rng(seed_of(w.cid, 0, 0, 0, "mask"))
    pairs = rng.choice(w.layers * w.H_kv, size=count, replace=False)
    for b in range(w.batch):
        for p in pairs:
            layer, head = divmod(int(p), w.H_kv)
            mask[(b * w.layers + layer) * w.H_kv + head] = 1
    return mask


def ar1_numpy(rng, T, d, rho, sigma, mu=None):
    """fp64 AR(1) sequence [T, d] with a plain loop (small sizes only)."""
    k = np.empty((T, d))
    k[0] = rng.standard_normal(d)
    for t in range(1, T):
        k[t] = rho * k[t - 1] + sigma * rng.standard_normal(d)
    if mu is not None:
        k = k + mu
    return k


def _ar1_scan_torch(x, rho):
    """y_t = rho * y_{t-1} + x_t along dim 1 of x [S, T, d] (fp32), blocked in time."""
    import torch
    S, T, d = x.shape
    Bk = 1
    while Bk * Bk < T:
        Bk *= 2
    nb = (T + Bk - 1) // Bk
    pad = nb * Bk - T
    if pad:
        x = torch.cat([x, x.new_zeros(S, pad, d)], dim=1)
    xb = x.view(S, nb, Bk, d)
    y = torch.empty_like(xb)
    r = rho.view(S, 1, 1)
    y[:, :, 0] = xb[:, :, 0]
    for t in range(1, Bk):
        y[:, :, t] = r * y[:, :, t - 1] + xb[:, :, t]
    pw = rho.view(S, 1) ** torch.arange(1, Bk + 1, device=x.device, dtype=x.dtype).view(1, Bk)
    for b in range(1, nb):
        y[:, b] += pw.view(S, Bk, 1) * y[:, b - 1, Bk - 1].view(S, 1, d)
    return y.view(S, nb * Bk, d)[:, :T]


def _torch_dtype(w):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]


def make_cache(w, device, ctx=None, batch_slices=32, with_appends=True):
    """Generate a whole cache for workload w on a torch device.

    Returns a dict of tensors: K, V [S, cap, d] in the storage type; N [S, cap] int32
    (1 for the first ctx rows, 0 beyond); lens [S] int32; mask [S] uint8;
    app_k, app_v [steps, S, d] (appended decode tokens) when w.append and with_appends.
    """
    import torch
    ctx = w.ctx if ctx is None else ctx
    S, cap, d = w.slices, w.cap - w.ctx + ctx, w.d
    dt = _torch_dtype(w)
    n_app = w.steps if (w.append and with_appends) else 0
    K = torch.zeros((S, cap, d), dtype=dt, device=device)
    V = torch.zeros((S, cap, d), dtype=dt, device=device)
    N = torch.zeros((S, cap), dtype=torch.int32, device=device)
    N[:, :ctx] = 1
    lens = torch.full((S,), ctx, dtype=torch.int32, device=device)
    app_k = torch.zeros((n_app, S, d), dtype=dt, device=device) if n_app else None
    app_v = torch.zeros((n_app, S, d), dtype=dt, device=device) if n_app else None
    T = ctx + n_app
    for z0 in range(0, S, batch_slices):
        zs = list(range(z0, min(S, z0 + batch_slices)))
        eps = torch.empty((len(zs), T, d), dtype=torch.float32, device=device)
        rho = torch.empty(len(zs), dtype=torch.float32, device=device)
        sig = torch.empty(len(zs), dtype=torch.float32, device=device)
        mus = torch.zeros((len(zs), 1, d), dtype=torch.float32, device=device)
        for i, z in enumerate(zs):
            b, layer, head = _slice_coords(w, z)
            gen = torch.Generator(device=device)
            gen.manual_seed(seed_of(w.cid, b, layer, head, "K"))
            eps[i] = torch.randn((T, d), generator=gen, device=device, dtype=torch.float32)
            r_, s_, mu = slice_params(w, z)
            rho[i], sig[i] = r_, s_
            if mu is not None:
                mus[i, 0] = torch.as_tensor(mu, dtype=torch.float32, device=device)
        eps[:, 1:] *= sig.view(-1, 1, 1)
        keys = _ar1_scan_torch(eps, rho) + mus
        del eps
        vals = torch.empty((len(zs), T, d), dtype=torch.float32, device=device)
        for i, z in enumerate(zs):
            b, layer, head = _slice_coords(w, z)
            gen = torch.Generator(device=device)
            gen.manual_seed(seed_of(w.cid, b, layer, head, "V"))
            vals[i] = torch.randn((T, d), generator=gen, device=device, dtype=torch.float32)
        K[z0:z0 + len(zs), :ctx] = keys[:, :ctx].to(dt)
        V[z0:z0 + len(zs), :ctx] = vals[:, :ctx].to(dt)
        if n_app:
            app_k[:, z0:z0 + len(zs)] = keys[:, ctx:].transpose(0, 1).to(dt)
            app_v[:, z0:z0 + len(zs)] = vals[:, ctx:].transpose(0, 1).to(dt)
        del keys, vals
    mask = torch.as_tensor(outlier_mask(w), device=device)
    out = {"K": K, "V": V, "N": N, "lens": lens, "mask": mask}
    if n_app:
        out["app_k"], out["app_v"] = app_k, app_v
    return out


def make_queries(w, device, steps=None):
    """q [steps, groups, H_q, d] ~ N(0, 1) in the storage type."""
    import torch
    steps = w.steps if steps is None else steps
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(w.cid, 0, 0, 0, "q"))
    q = torch.randn((steps, w.groups, w.H_q, w.d), generator=gen, device=device,
                    dtype=torch.float32)
    return q.to(_torch_dtype(w))
