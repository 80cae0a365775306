"""Seeded synthetic inputs for the GCA hot path.

This module only draws random numbers and lays them out; it holds none of
GCA's arithmetic.  Both the GPU library's tests/benchmark and the float64
oracle consume what it returns.  The workloads stand in for the pages' data
(PG19 / arXiv-math training at 16K tokens, needle-in-a-haystack up to 16M
tokens), which is not available here: only shapes, value distributions and
structure are reproduced.

Draws use numpy's PCG64 with SeedSequence(seed).spawn(8) sub-streams in the fixed
order  q, k, v, landmarks, dout, needle positions, query landmarks, redraws.
bf16 inputs are drawn in float32 and rounded to nearest-even by torch's CPU
cast; the stored (rounded) values are the inputs of both sides.

Tie avoidance: a caller may pass `accept(lq_rows, lk_rows, n_cand)` returning
one boolean per query row; rejected query landmarks are redrawn from the
"redraws" sub-stream (in a fixed order) until accepted.  The predicate itself
lives with the test code.
"""

import math

import numpy as np
import torch

__all__ = ["WORKLOADS", "workload", "training_inputs", "context_landmarks",
           "device_kv", "query_batch", "kv_tiles_host", "SWA_WORKLOADS", "swa_inputs"]

# Sizes of each workload, named by what it is.
WORKLOADS = {
    # fp32, 256 tokens = 16 chunks of 16, landmark/head dim 32, top-2, vanilla.
    "tiny_fp32": dict(G=1, B=1, H=2, n_query=16, n_key=16, S=16, D=32, Dl=32,
                      k=2, dtype="f32", softmax_one=0, landmarks="aliased",
                      value_scale=1.0, seed=1),
    # bf16, 16384 tokens = 256 chunks of 64, top-8, one group, vanilla.
    "train16k_fwd": dict(G=1, B=4, H=12, n_query=256, n_key=256, S=64, D=64,
                         Dl=64, k=8, dtype="bf16", softmax_one=0,
                         landmarks="aliased", value_scale=0.125, seed=2),
    # bf16 training step of one upper layer: two groups, off-by-one weights.
    "train16k_fwdbwd_g2": dict(G=2, B=4, H=12, n_query=256, n_key=256, S=64,
                               D=64, Dl=64, k=8, dtype="bf16", softmax_one=1,
                               landmarks="separate", value_scale=0.125, seed=3),
    # bf16 inference step over a resident 1,048,576-token context: one new
    # query chunk against 16384 resident chunks (16383 candidates).
    "infer1m_step": dict(G=1, B=1, H=12, n_query=1, n_key=16384, S=64, D=64,
                         Dl=64, k=8, dtype="bf16", softmax_one=0,
                         landmarks="needle", value_scale=0.125, seed=4,
                         q_pos=16384, steps=1000),
    # bf16 retrieval over a resident 16,777,216-token context: 32 query chunks
    # against all 262144 resident chunks.
    "retrieve16m": dict(G=1, B=1, H=12, n_query=32, n_key=262144, S=64, D=64,
                        Dl=64, k=8, dtype="bf16", softmax_one=0,
                        landmarks="needle", value_scale=0.125, seed=5,
                        q_pos=262145),
}

_STREAMS = ("q", "k", "v", "landmarks", "dout", "needle", "qland", "redraw")
NEEDLE_COS = 0.9


def workload(name, **override):
    w = dict(WORKLOADS[name])
    w.update(override)
    w["name"] = name
    w.setdefault("attn_scale", 1.0 / math.sqrt(w["D"]))
    w.setdefault("score_scale", 1.0 / math.sqrt(w["Dl"]))
    return w


def _streams(seed):
    seqs = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(_STREAMS, seqs)}


def _stored(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _normal(rng, shape, scale, dtype):
    return _stored(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale), dtype)


def _f64(t):
    return t.to(torch.float64).numpy()


def _q_pos_training(n_query):
    return torch.arange(n_query, dtype=torch.int32)


def training_inputs(name, seed=None, accept=None, with_dout=True, **override):
    """Inputs of a training-shaped workload (query chunks == key chunks).

    Returns a dict of CPU tensors q, k, v, lq, lk, q_pos, dout plus "cfg".
    Landmarks: "aliased" draws one landmark per chunk l and sets lq[t] = l[t-1]
    (lq[0] = 0), lk = l; "separate" draws lq and lk independently per group.
    """
    cfg = workload(name, **override)
    if seed is None:
        seed = cfg["seed"]
    rs = _streams(seed)
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, dt, sc = cfg["S"], cfg["D"], cfg["Dl"], cfg["dtype"], cfg["value_scale"]
    q = _normal(rs["q"], (G, B, H, Nq, S, D), sc, dt)
    k = _normal(rs["k"], (G, B, H, Nk, S, D), sc, dt)
    v = _normal(rs["v"], (G, B, H, Nk, S, D), sc, dt)
    q_pos = _q_pos_training(Nq)
    heads = [(g, b, h) for g in range(G) for b in range(B) for h in range(H)]
    if cfg["landmarks"] == "aliased":
        assert Nq == Nk
        l = _normal(rs["landmarks"], (G, B, H, Nk, Dl), sc, dt)
        if accept is not None:
            l64 = _f64(l)
            for t in range(2, Nq):
                n = t - 1  # query t uses l[t-1]; candidates l[0..t-2]
                if n <= cfg["k"]:
                    continue
                while True:
                    rows = np.stack([l64[g, b, h, t - 1] for (g, b, h) in heads])
                    cands = np.stack([l64[g, b, h, :n] for (g, b, h) in heads])
                    ok = accept(rows, cands, np.full(len(heads), n))
                    if ok.all():
                        break
                    for j in np.flatnonzero(~ok):
                        g, b, h = heads[j]
                        new = _normal(rs["redraw"], (Dl,), sc, dt)
                        l[g, b, h, t - 1] = new
                        l64[g, b, h, t - 1] = _f64(new)
        lk = l.clone()
        lq = torch.zeros_like(l)
        lq[:, :, :, 1:] = l[:, :, :, :-1]
    else:
        lq = _normal(rs["qland"], (G, B, H, Nq, Dl), sc, dt)
        lk = _normal(rs["landmarks"], (G, B, H, Nk, Dl), sc, dt)
        if accept is not None:
            lk64 = _f64(lk)
            lq64 = _f64(lq)
            for (g, b, h) in heads:
                todo = np.array([t for t in range(Nq) if t - 1 > cfg["k"]])
                while todo.size:
                    n = todo - 1
                    ok = accept(lq64[g, b, h, todo], np.broadcast_to(
                        lk64[g, b, h], (todo.size, Nk, Dl)), n)
                    for t in todo[~ok]:
                        new = _normal(rs["redraw"], (Dl,), sc, dt)
                        lq[g, b, h, t] = new
                        lq64[g, b, h, t] = _f64(new)
                    todo = todo[~ok]
    out = dict(q=q, k=k, v=v, lq=lq, lk=lk, q_pos=q_pos, cfg=cfg)
    if with_dout:
        out["dout"] = _stored(rs["dout"].standard_normal((G, B, H, Nq, S, D),
                                                         dtype=np.float32), dt)
    return out


def context_landmarks(name, seed=None, **override):
    """Resident landmarks lk [G, B, H, Nk, Dl] of a long-context workload (CPU)."""
    cfg = workload(name, **override)
    if seed is None:
        seed = cfg["seed"]
    rs = _streams(seed)
    G, B, H, Nk, Dl = cfg["G"], cfg["B"], cfg["H"], cfg["n_key"], cfg["Dl"]
    return _normal(rs["landmarks"], (G, B, H, Nk, Dl), cfg["value_scale"], cfg["dtype"])


def device_kv(name, device, seed=None, slice_chunks=8192, **override):
    """Resident K and V [G, B, H, Nk, S, D] drawn directly in device memory.

    Drawn slice by slice with a seeded torch generator on the device (N(0,1)
    times value_scale, rounded to bf16), so that tens of GB never pass through
    host memory.  `kv_tiles_host` copies selected tiles back for the oracle.
    """
    cfg = workload(name, **override)
    if seed is None:
        seed = cfg["seed"]
    G, B, H, Nk, S, D = cfg["G"], cfg["B"], cfg["H"], cfg["n_key"], cfg["S"], cfg["D"]
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    outs = []
    for _ in range(2):
        t = torch.empty((G, B, H, Nk, S, D), dtype=dt, device=device)
        flat = t.view(G * B * H, Nk, S, D)
        for hh in range(G * B * H):
            for c0 in range(0, Nk, slice_chunks):
                c1 = min(Nk, c0 + slice_chunks)
                x = torch.randn((c1 - c0, S, D), generator=gen, device=device,
                                dtype=torch.float32)
                flat[hh, c0:c1] = (x * cfg["value_scale"]).to(dt)
        outs.append(t)
    return outs[0], outs[1]


def kv_tiles_host(t, chunks):
    """Host float64 copy of the listed chunk tiles of a device K or V tensor.

    Returns {(g, b, h, c): [S, D] array}."""
    out = {}
    for key in chunks:
        g, b, h, c = key
        out[key] = t[g, b, h, c].to("cpu").to(torch.float64).numpy()
    return out


def query_batch(name, lk, step=0, seed=None, accept=None, accept_heads=None, lk64=None,
                **override):
    """Query chunks of a long-context workload with one planted needle each.

    For query chunk n the needle is resident chunk needle[n] (distinct per
    query, the same in every head); its query landmark in every head is
      lq = |g| (0.9 u + sqrt(1 - 0.81) v)
    with u the unit needle landmark, v a random unit vector orthogonal to u and
    |g| the norm of a fresh N(0, value_scale^2) draw, rounded to the stored dtype.
    `accept_heads` (list of (g, b, h)) limits the redraw rule to those heads.
    `lk64` may pass a float64 copy of lk (reused across many steps).
    Returns dict q [G,B,H,Nq,S,D], lq [G,B,H,Nq,Dl], q_pos [Nq], needle [Nq].
    """
    cfg = workload(name, **override)
    if seed is None:
        seed = cfg["seed"]
    rs = _streams([int(seed), int(step)])
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, dt, sc = cfg["S"], cfg["D"], cfg["Dl"], cfg["dtype"], cfg["value_scale"]
    q_pos_val = cfg["q_pos"]
    n_cand = max(0, min(q_pos_val - 1, Nk))
    needle = rs["needle"].choice(n_cand, size=Nq, replace=False)
    q = _normal(rs["q"], (G, B, H, Nq, S, D), sc, dt)
    if lk64 is None:
        lk64 = _f64(lk)

    def draw(g, b, h, n, rng):
        u = lk64[g, b, h, needle[n]]
        u = u / np.linalg.norm(u)
        r = rng.standard_normal(Dl)
        r -= u * float(r @ u)
        r /= np.linalg.norm(r)
        mag = np.linalg.norm(rng.standard_normal(Dl) * sc)
        vec = mag * (NEEDLE_COS * u + math.sqrt(1.0 - NEEDLE_COS ** 2) * r)
        return _stored(vec[None, :], dt)[0]

    lq = torch.empty((G, B, H, Nq, Dl), dtype=q.dtype)
    for g in range(G):
        for b in range(B):
            for h in range(H):
                for n in range(Nq):
                    lq[g, b, h, n] = draw(g, b, h, n, rs["qland"])
    if accept is not None:
        for g in range(G):
            for b in range(B):
                for h in range(H):
                    if accept_heads is not None and (g, b, h) not in accept_heads:
                        continue
                    todo = np.arange(Nq)
                    while todo.size:
                        ok = accept(_f64(lq[g, b, h, todo]), lk64[g, b, h, :n_cand],
                                    np.full(todo.size, n_cand))
                        for n in todo[~ok]:
                            lq[g, b, h, n] = draw(g, b, h, n, rs["redraw"])
                        todo = todo[~ok]
    q_pos = torch.full((Nq,), q_pos_val, dtype=torch.int32)
    return dict(q=q, lq=lq, q_pos=q_pos, needle=torch.from_numpy(needle), cfg=cfg)


# Sliding-window self-attention of the same layer: the 16K-token training batch
# (B=4, H=12, 16384 tokens, head dim 64) with the pages' 512-token window.
SWA_WORKLOADS = {
    "train16k_swa": dict(B=4, H=12, T=16384, D=64, window=512, seed=6),
}


def swa_inputs(B, H, T, D, seed, device="cpu"):
    """q, k, v, dout [B, H, T, D] bf16, N(0, 1) each (so that scale * <q, k> has
    unit spread at scale 1/sqrt(D)).  Large sizes are drawn on `device` with a
    seeded torch generator, one tensor at a time; small ones (device "cpu")
    from numpy's PCG64 sub-streams q, k, v, dout."""
    if device == "cpu":
        rs = _streams(seed)
        return {name: _normal(rs[name], (B, H, T, D), 1.0, "bf16")
                for name in ("q", "k", "v", "dout")}
    g = torch.Generator(device=device)
    out = {}
    for i, name in enumerate(("q", "k", "v", "dout")):
        g.manual_seed(seed * 16 + i)
        out[name] = torch.randn((B, H, T, D), generator=g, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out
