"""Benchmark of the GCA hot path on one MI355X.

One step = one training pass of one upper layer's Grouped Cross Attention over
a 16K-token batch: gca_retrieve (landmark scan, top-8, fusion weights) +
gca_forward (per-chunk attention and fusion) + gca_backward (dQ, dK, dV, dw,
dscore, d landmarks), for G=2 retrieval groups with softmax off-by-one, B=4,
H=12, 16384 tokens = 256 chunks of 64, head/landmark dim 64, bf16 inputs with
float32 accumulation.  Inputs are seeded synthetic tensors resident in HBM.

Prints ONE JSON line: tokens/s of the whole step, the roofline position of the
dominant kernel (per-kernel HIP-event timing inside the timed region) and the
float64 oracle timed on a bounded sample on the host cores.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--cpu-heads N]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
MFMA_BF16_PEAK = 2.5e15    # MI355X dense bf16 MFMA, flop/s
WORKLOAD = "train16k_fwdbwd_g2"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the 16M-token retrieval and 1M-token inference measurements")
    ap.add_argument("--infer-steps", type=int, default=1000)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cold-cache step, the copy rate, the one-group forward and "
                         "the step at the other tile sizes")
    ap.add_argument("--no-swa", action="store_true",
                    help="skip the sliding-window self-attention step")
    ap.add_argument("--no-gumbel", action="store_true",
                    help="skip the training step with Gumbel top-k retrieval")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="BYTES",
                    help="after the timed steps, one device-to-device copy of BYTES "
                         "(reference dispatch for scaling hardware byte counters)")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "retrieval_sparse_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_work(cfg, pairs):
    """Algorithmic HBM bytes and flops of one launch of each kernel.

    Bytes count every tensor the kernel must read or write once (gathered K/V
    tiles that are re-read from cache are not counted again); flops count the
    tile products the kernel must form given its inputs (2*S*S*D each).
    """
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, k = cfg["S"], cfg["D"], cfg["Dl"], cfg["k"]
    heads = G * B * H
    tile = S * D * 2                       # one bf16 chunk tile
    qt, kt = heads * Nq * tile, heads * Nk * tile
    slots = heads * Nq * k
    mm = 2 * S * S * D                      # one S x S x D product
    cand = heads * sum(max(0, min(t - 1, Nk)) for t in range(Nq))
    return {
        "scan_topk": dict(bytes=heads * (Nq + Nk) * Dl * 2 + slots * 12 + Nq * 4,
                          flops=2 * Dl * cand),
        "forward": dict(bytes=qt + 2 * kt + qt + slots * S * 4 + slots * 8,
                        flops=2 * mm * pairs),
        "reverse_index": dict(bytes=slots * 8 + heads * (Nk + 1) * 4, flops=0),
        "backward_q": dict(bytes=2 * qt + 2 * kt + qt + 2 * slots * S * 4 + slots * 16
                           + heads * Nq * Dl * 4, flops=3 * mm * pairs),
        "backward_kv": dict(bytes=2 * kt + 2 * qt + 2 * kt + 2 * slots * S * 4 + slots * 12
                            + heads * Nk * Dl * 4, flops=4 * mm * pairs),
    }


def step_work(cfg, pairs):
    """Algorithmic HBM bytes and flops of one whole training step: every input
    read once and every output written once (forward: q, k, v, landmarks, idx, w
    in, o and lse out; backward: q, k, v, dO, lse, idx, w, landmarks in, dq, dk,
    dv, dw, dscore, dlq, dlk out), and 2 forward plus 5 backward tile products
    per (query chunk, retrieved chunk) pair."""
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, k = cfg["S"], cfg["D"], cfg["Dl"], cfg["k"]
    heads = G * B * H
    tile = S * D * 2
    qt, kt = heads * Nq * tile, heads * Nk * tile
    slots = heads * Nq * k
    land = heads * (Nq + Nk) * Dl * 2
    retrieve = land + slots * 12
    fwd = qt + 2 * kt + slots * 8 + qt + slots * S * 4
    bwd = (2 * qt + 2 * kt + slots * S * 4 + slots * 8 + land + qt + 2 * kt + slots * 8
           + heads * (Nq + Nk) * Dl * 4)
    return {"bytes": retrieve + fwd + bwd, "flops": 7 * 2 * S * S * D * pairs}


def roofline_entry(name, avg_s, work):
    t_hbm = work["bytes"] / HBM_PEAK
    t_mfma = work["flops"] / MFMA_BF16_PEAK
    if t_mfma >= t_hbm:
        ach = work["flops"] / avg_s / 1e12
        return dict(kernel=name, bound="mfma", achieved=round(ach, 2),
                    peak=MFMA_BF16_PEAK / 1e12, unit="TFLOP/s",
                    frac=round(ach / (MFMA_BF16_PEAK / 1e12), 4))
    ach = work["bytes"] / avg_s / 1e9
    return dict(kernel=name, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK / 1e9,
                unit="GB/s", frac=round(ach / (HBM_PEAK / 1e9), 4))


def measure_peaks(reps=10):
    """Peaks of the GPU at hand, from the microbenchmarks built into the library
    (include/gca_peaks.h): a streaming read of 2 GiB, a 1 GiB device copy and a loop
    of independent 16x16x32 bf16 MFMAs; median of reps launches each (HIP events)."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as gca
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    out = torch.empty(gca.PEAK_OUT_BYTES, dtype=torch.uint8, device="cuda")
    n_read, n_copy = 2 << 30, 1 << 30
    src = torch.ones(n_read, dtype=torch.uint8, device="cuda")
    t_read = timed(lambda: gca.gca_peak_read(src, out))
    dst = torch.empty(n_copy, dtype=torch.uint8, device="cuda")
    t_copy = timed(lambda: gca.gca_peak_copy(src[:n_copy], dst))
    mf = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    flops = [0.0]

    def mfma():
        flops[0] = gca.gca_peak_mfma(mf, 2048)

    t_mfma = timed(mfma)
    # tile gathers into LDS from a buffer that every XCD's L2 holds (2 MiB), one that
    # only the last-level cache holds (32 MiB) and one from HBM (1 GiB)
    gout = torch.empty(gca.PEAK_GATHER_OUT_BYTES, dtype=torch.uint8, device="cuda")
    moved = [0.0]
    gather = {}
    for label, size, iters in (("l2", 2 << 20, 64), ("llc", 32 << 20, 16), ("hbm", 1 << 30, 16)):
        def gfn(size=size, iters=iters):
            moved[0] = gca.gca_peak_gather(src[:size], gout, iters)
        t = timed(gfn)
        gather[f"gather_{label}_GBps"] = round(moved[0] / t / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(n_read / t_read / 1e9, 1),
            "copy_read_plus_write_GBps": round(2 * n_copy / t_copy / 1e9, 1),
            "mfma_bf16_dense_TFLOPs": round(flops[0] / t_mfma / 1e12, 1),
            **gather,
            "note": "gca_peak_read (2 GiB), gca_peak_copy (1 GiB), gca_peak_mfma (16x16x32 "
                    "bf16, 4 waves per SIMD, 8 independent accumulators per wave), "
                    "gca_peak_gather (random 16 KB tiles into LDS, one in flight per "
                    "workgroup, 4 workgroups per CU; from 2 MiB, 32 MiB and 1 GiB buffers)"}


def with_measured(entry, peaks):
    """Adds the fraction of the measured peak of the entry's bound to a roofline entry."""
    if peaks is None:
        return entry
    mp = peaks["hbm_read_GBps"] if entry["bound"] == "hbm" else peaks["mfma_bf16_dense_TFLOPs"]
    entry["measured_peak"] = mp
    entry["frac_of_measured_peak"] = round(entry["achieved"] / mp, 4)
    return entry


def traffic_for(kernel, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}@{WORKLOAD}")
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# CPU baseline: the float64 oracle, timed on the host cores beside the GPU run.
# Its inputs are generated before anything touches the GPU and a pool of
# worker processes is forked then, so the workers share the inputs and never
# inherit GPU state.  Each worker runs the oracle with BLAS on one thread.
# --------------------------------------------------------------------------
_CPU = {}  # inputs the oracle workers read (filled before the pool is forked)


def cpu_workers():
    """Oracle worker processes: the cores this process may use, at most 16
    (OMP_NUM_THREADS when set, e.g. a one-GPU share of a larger host)."""
    n = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(n, cap, 16))


def _worker_init():
    from threadpoolctl import threadpool_limits
    global _BLAS_LIMIT
    _BLAS_LIMIT = threadpool_limits(1)


class _HostTiles:
    """K or V of one head at a long context, for the oracle: chunk c's tile is
    pool[(salt + 7919 c) mod len(pool)], a pool of host-drawn N(0,1)/8 tiles
    rounded to bf16 (the device-drawn K/V are never copied back).  The oracle
    only indexes it by chunk and reads its length."""

    def __init__(self, pool, n_key, salt):
        self.pool, self.salt = pool, salt
        self.shape = (n_key,) + tuple(pool.shape[1:])

    def __getitem__(self, c):
        return self.pool[(self.salt + 7919 * int(c)) % self.pool.shape[0]]


def _tile_pool(S, D, seed, n=512):
    import numpy as np
    import torch
    rng = np.random.default_rng(seed)
    t = torch.from_numpy((rng.standard_normal((n, S, D)) / 8).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _cpu_job(job):
    """One oracle job in a worker; returns the number of units it did."""
    from oracle import gca_oracle as orc
    kind, arg = job
    f = lambda t: t.to("cpu").double().numpy()
    if kind in ("train", "fwd"):
        d = _CPU[kind]
        x, cfg = d["x"], d["cfg"]
        for (g, b, h) in arg:
            sl = lambda t: f(t[g:g + 1, b:b + 1, h:h + 1])
            q, k, v, lq, lk = sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["lq"]), sl(x["lk"])
            idx, _, w = orc.retrieve(lq, lk, x["q_pos"].numpy(), cfg["k"], cfg["score_scale"],
                                     cfg["softmax_one"])
            orc.forward(q, k, v, idx, w, cfg["attn_scale"])
            if kind == "train":
                orc.backward(q, k, v, idx, w, sl(x["dout"]), lq, lk, cfg["attn_scale"],
                             cfg["score_scale"])
        return len(arg)
    if kind == "infer1m":
        d = _CPU[kind]
        cfg, lk = d["cfg"], d["lk"]
        H = cfg["H"]
        lk64 = [f(lk[0, 0, h]) for h in range(H)]
        kt = [_HostTiles(d["kpool"], cfg["n_key"], 11 * h) for h in range(H)]
        vt = [_HostTiles(d["vpool"], cfg["n_key"], 13 * h + 5) for h in range(H)]
        q_pos = int(d["q_pos"])
        for s in arg:
            for h in range(H):
                lq_row = f(d["lqs"][s, 0, 0, h, 0])
                idx, _, w = orc.retrieve_one(lq_row, lk64[h], q_pos, cfg["k"],
                                             cfg["score_scale"], cfg["softmax_one"])
                orc.forward_query_chunk(f(d["qs"][s, 0, 0, h, 0]), kt[h], vt[h], idx, w,
                                        cfg["attn_scale"])
        return len(arg)
    if kind == "retrieve16m":
        d = _CPU[kind]
        cfg, h = d["cfg"], arg
        lk64 = f(d["lk"][0, 0, h])
        kt = _HostTiles(d["kpool"], cfg["n_key"], 11 * h)
        vt = _HostTiles(d["vpool"], cfg["n_key"], 13 * h + 5)
        q_pos = int(d["q_pos"][0])
        for n in range(cfg["n_query"]):
            idx, _, w = orc.retrieve_one(f(d["lq"][0, 0, h, n]), lk64, q_pos, cfg["k"],
                                         cfg["score_scale"], cfg["softmax_one"])
            orc.forward_query_chunk(f(d["q"][0, 0, h, n]), kt, vt, idx, w, cfg["attn_scale"])
        return cfg["n_query"]
    raise ValueError(kind)


def _run_jobs(pool, jobs):
    t0 = time.perf_counter()
    units = sum(pool.map(_cpu_job, jobs, chunksize=1))
    return time.perf_counter() - t0, units


def _split(items, n):
    n = max(1, min(n, len(items)))
    return [items[i::n] for i in range(n)]


def cpu_baselines(pool, workers):
    """The oracle on each measured workload, all workers; one dict per workload."""
    out = {}
    blas = "BLAS limited to 1 thread per worker process"
    if "train" in _CPU:
        cfg = _CPU["train"]["cfg"]
        heads = [(g, b, h) for g in range(cfg["G"]) for b in range(cfg["B"])
                 for h in range(cfg["H"])]
        parts = _split(heads, workers)
        dt, n = _run_jobs(pool, [("train", p) for p in parts])
        tokens = cfg["B"] * cfg["n_query"] * cfg["S"]
        out["train"] = dict(value=round(tokens / dt, 2), unit="tokens/s", cores=len(parts),
                            kind="oracle", blas_threads=1,
                            sample=f"the whole step: all {n} (g,b,h) heads, retrieve + forward + "
                                   f"backward, float64 numpy, {len(parts)} worker processes, "
                                   f"{blas}; {dt:.2f} s wall")
    if "fwd" in _CPU:
        cfg = _CPU["fwd"]["cfg"]
        heads = [(g, b, h) for g in range(cfg["G"]) for b in range(cfg["B"])
                 for h in range(cfg["H"])]
        parts = _split(heads, workers)
        dt, n = _run_jobs(pool, [("fwd", p) for p in parts])
        tokens = cfg["B"] * cfg["n_query"] * cfg["S"]
        out["fwd"] = dict(value=round(tokens / dt, 2), unit="tokens/s", cores=len(parts),
                          kind="oracle", blas_threads=1,
                          sample=f"all {n} (g,b,h) heads, retrieve + forward, float64 numpy, "
                                 f"{len(parts)} worker processes, {blas}; {dt:.2f} s wall")
    if "infer1m" in _CPU:
        steps = list(range(_CPU["infer1m"]["lqs"].shape[0]))
        parts = _split(steps, workers)
        dt, n = _run_jobs(pool, [("infer1m", p) for p in parts])
        out["infer1m"] = dict(value=round(n / dt, 2), unit="steps/s", cores=len(parts),
                              kind="oracle", blas_threads=1,
                              us_per_step_amortised=round(dt / n * 1e6, 1),
                              sample=f"all {n} chunk steps x 12 heads (scan of 16383 landmarks, "
                                     f"top-8, 8-chunk attention), steps split over "
                                     f"{len(parts)} worker processes, {blas}; K/V tiles drawn "
                                     f"on the host (same distribution); {dt:.2f} s wall")
    if "retrieve16m" in _CPU:
        H = _CPU["retrieve16m"]["cfg"]["H"]
        jobs = [("retrieve16m", h) for h in range(H)]
        dt, n = _run_jobs(pool, jobs)
        out["retrieve16m"] = dict(value=round(dt * 1e3, 2), unit="ms (retrieve + forward)",
                                  cores=min(workers, H), kind="oracle", blas_threads=1,
                                  sample=f"the whole batch: {n} query chunks x 262144 resident "
                                         f"chunks, one worker process per head ({H} heads on "
                                         f"{min(workers, H)} workers), {blas}; K/V tiles drawn "
                                         f"on the host (same distribution); {dt:.2f} s wall")
    return out


def _latency(fn, reps):
    """Average ms of fn() over reps calls on the current stream, with the library's
    per-kernel event timing off."""
    import torch

    import retrieval_sparse_attention_amd as gca
    gca.gca_timing_enable(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _timed(fn, reps):
    """Average ms of fn() over reps calls, on the current stream, plus per-kernel sums."""
    import torch

    import retrieval_sparse_attention_amd as gca
    gca.gca_timing_enable(True)
    gca.gca_timing_collect()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    gca.gca_timing_enable(False)
    per = {k: v[0] / v[1] for k, v in gca.gca_timing_collect().items() if v[1]}
    return e0.elapsed_time(e1) / reps, per


def bench_gumbel_step(shape, d, bufs, steps):
    """The same training step with gca_retrieve_gumbel (a fresh seed per step,
    as in training) in place of gca_retrieve."""
    import retrieval_sparse_attention_amd as gca
    idx, score, w, o, lse, dq, dk, dv, dw, dscore, dlq, dlk, wsr, wsb = bufs
    seed = [1000]

    def step():
        seed[0] += 1
        gca.gca_retrieve_gumbel(shape, seed[0], d["lq"], d["lk"], d["q_pos"], idx, score, w,
                                ws=wsr)
        gca.gca_forward(shape, d["q"], d["k"], d["v"], idx, w, o, lse)
        gca.gca_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"],
                         dq, dk, dv, dw, dscore, dlq, dlk, ws=wsb)

    for _ in range(3):
        step()
    ms = _latency(step, steps)  # per-kernel events off, as for the headline
    _, per = _timed(step, steps)
    tokens = shape.B * shape.n_query * shape.chunk_size
    return {"retrieval": "gca_retrieve_gumbel (Philox4x32-10 Gumbel noise, new seed per step)",
            "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 4), "steps": steps,
            "scan_us": round(per.get("scan_topk", 0.0) * 1e3, 2),
            "kernels_us": {key: round(val * 1e3, 2) for key, val in per.items()}}


def swa_pairs(T, W):
    """(query, key) pairs inside a causal window of W over T tokens."""
    W = min(W, T)
    return W * (W + 1) // 2 + (T - W) * W


def bench_swa(steps):
    """Sliding-window self-attention of the same layer over the 16K-token
    batch (B=4, H=12, T=16384, D=64, W=512): forward + backward per step."""
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    cfg = synth.SWA_WORKLOADS["train16k_swa"]
    B, H, T, D, W = cfg["B"], cfg["H"], cfg["T"], cfg["D"], cfg["window"]
    x = synth.swa_inputs(B, H, T, D, cfg["seed"], device="cuda")
    shape = gca.make_swa_shape(B, H, T, D, W)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
    ws = torch.empty(gca.gca_swa_workspace_size(shape), dtype=torch.uint8, device="cuda")

    def step():
        gca.gca_swa_forward(shape, x["q"], x["k"], x["v"], o, lse)
        gca.gca_swa_backward(shape, x["q"], x["k"], x["v"], o, lse, x["dout"], dq, dk, dv, ws=ws)

    for _ in range(3):
        step()
    ms = _latency(step, steps)  # step time with the per-kernel events off
    _, per = _timed(step, steps)
    pairs = B * H * swa_pairs(T, W)
    # algorithmic flops over the pairs inside the window: 2 products (QK, PV)
    # forward, 5 (QK, dO V^T, dQ, dK, dV) backward, 2*D flops each
    work = {"swa_forward": 2 * 2 * D * pairs, "swa_backward_q": 3 * 2 * D * pairs,
            "swa_backward_kv": 4 * 2 * D * pairs}
    kern = {}
    for name, f in work.items():
        t = per.get(name)
        if t:
            tf = f / (t * 1e-3) / 1e12
            kern[name] = dict(avg_us=round(t * 1e3, 2), tflops=round(tf, 1),
                              frac=round(tf / (MFMA_BF16_PEAK / 1e12), 4))
    tokens = B * T
    return {"workload": "train16k_swa", "B": B, "H": H, "tokens": T, "head_dim": D,
            "window": W, "step": "gca_swa_forward + gca_swa_backward", "steps": steps,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "pairs": pairs, "kernels": kern,
            "algorithmic_flops_per_step": 2 * D * pairs * (2 + 5),
            "note": "backward recomputes S and dP in both kernels (7 tile products per "
                    "pair instead of 5); flops above count the 5 the math needs"}


def bench_train16k_fwd(steps, x=None):
    """The 16K-token forward of one group (G=1, vanilla weights, aliased landmarks):
    gca_retrieve + gca_forward per step, against max(HBM, MFMA) time of the forward's
    algorithmic bytes and flops."""
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    name = "train16k_fwd"
    cfg = synth.workload(name)
    if x is None:
        x = synth.training_inputs(name, with_dout=False)
    d = {key: val.contiguous().cuda() for key, val in x.items() if key != "cfg"}
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, k = cfg["S"], cfg["D"], cfg["Dl"], cfg["k"]
    shape = gca.make_shape(G, B, H, Nq, Nk, S, D, Dl, k, gca.GCA_BF16, cfg["softmax_one"])
    idx = torch.empty((G, B, H, Nq, k), dtype=torch.int32, device="cuda")
    score = torch.empty((G, B, H, Nq, k), device="cuda")
    w = torch.empty_like(score)
    o = torch.empty_like(d["q"])
    lse = torch.empty((G, B, H, Nq, k, S), device="cuda")

    def step():
        gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], idx, score, w)
        gca.gca_forward(shape, d["q"], d["k"], d["v"], idx, w, o, lse)

    for _ in range(3):
        step()
    ms = _latency(step, steps)  # step time with the per-kernel events off
    _, per = _timed(step, steps)
    pairs = int((idx >= 0).sum().item())
    wk = kernel_work(cfg, pairs)["forward"]
    fwd_s = per.get("forward", 0.0) * 1e-3
    t_roof = max(wk["bytes"] / HBM_PEAK, wk["flops"] / MFMA_BF16_PEAK)
    return {"workload": name, "G": G, "B": B, "H": H, "tokens": Nq * S, "pairs": pairs,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * Nq * S / (ms / 1e3), 1),
            "forward_us": round(fwd_s * 1e6, 2), "scan_us": round(per.get("scan_topk", 0.0) * 1e3, 2),
            "forward_GBps": round(wk["bytes"] / fwd_s / 1e9, 1) if fwd_s else None,
            "forward_TFLOPs": round(wk["flops"] / fwd_s / 1e12, 1) if fwd_s else None,
            "forward_roofline_us": round(t_roof * 1e6, 2),
            "forward_roofline_frac": round(t_roof / fwd_s, 4) if fwd_s else None}


def bench_tile_sizes(steps):
    """The training step of the headline workload (retrieve + forward + backward, G=2, B=4,
    H=12, 16K tokens, k=8, off-by-one weights) at the other bf16 tile sizes that run on
    MFMA kernels: 64-token chunks with head_dim 32, and 16-token chunks with head_dim 64
    and 32 (n = 16384 / S chunks per head).  Tokens per step count B * 16K, as in the
    headline."""
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    out = {}
    for S, D in ((64, 32), (16, 64), (16, 32)):
        n = 16384 // S
        over = dict(S=S, D=D, n_query=n, n_key=n)
        cfg = synth.workload(WORKLOAD, **over)
        x = synth.training_inputs(WORKLOAD, **over)
        d = {key: val.contiguous().cuda() for key, val in x.items() if key != "cfg"}
        del x
        G, B, H, k, Dl = cfg["G"], cfg["B"], cfg["H"], cfg["k"], cfg["Dl"]
        shape = gca.make_shape(G, B, H, n, n, S, D, Dl, k, gca.GCA_BF16, cfg["softmax_one"])
        idx = torch.empty((G, B, H, n, k), dtype=torch.int32, device="cuda")
        score = torch.empty((G, B, H, n, k), device="cuda")
        w = torch.empty_like(score)
        o = torch.empty_like(d["q"])
        lse = torch.empty((G, B, H, n, k, S), device="cuda")
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        dw, dscore = torch.empty_like(w), torch.empty_like(w)
        dlq = torch.empty(tuple(d["lq"].shape), device="cuda")
        dlk = torch.empty(tuple(d["lk"].shape), device="cuda")
        wsr = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)),
                          dtype=torch.uint8, device="cuda")
        wsb = torch.empty(gca.gca_workspace_size(shape, gca.OP_BACKWARD), dtype=torch.uint8,
                          device="cuda")

        def step():
            gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], idx, score, w, ws=wsr)
            gca.gca_forward(shape, d["q"], d["k"], d["v"], idx, w, o, lse)
            gca.gca_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"],
                             d["lk"], dq, dk, dv, dw, dscore, dlq, dlk, ws=wsb)

        for _ in range(3):
            step()
        ms = _latency(step, steps)  # step time with the per-kernel events off
        _, per = _timed(step, steps)
        out[f"S{S}_D{D}"] = {"chunk_size": S, "head_dim": D, "chunks_per_head": n,
                             "ms_per_step": round(ms, 4),
                             "tokens_per_s": round(B * n * S / (ms / 1e3), 1),
                             "kernels_us": {kn: round(v * 1e3, 2) for kn, v in per.items()}}
        del d, o, lse, dq, dk, dv, wsr, wsb
        torch.cuda.empty_cache()
    return out


def bench_cold_and_copy(step, reps=5):
    """The training step "cold": a 512 MB buffer is written before each timed step so that
    the last-level cache (MALL) holds none of the inputs; plus the rate of a plain 1 GiB
    device-to-device copy, the HBM rate a streaming kernel reaches on this machine."""
    import numpy as np
    import torch
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold = []
    for r in range(reps):
        flush.fill_(float(r))
        torch.cuda.synchronize()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    src = torch.ones(2**30 // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 5 / 1e3
    del src, dst
    torch.cuda.empty_cache()
    return {"cold_ms_per_step_median": round(float(np.median(cold)), 4), "cold_reps": reps,
            "copy_1GiB_read_plus_write_GBps": round(2 * 2**30 / copy_s / 1e9, 1)}


def long_context_inputs(name, steps=1):
    """Resident landmarks and the query chunk batches (one per step) of a
    long-context workload, on the host."""
    import torch

    import synth
    lk = synth.context_landmarks(name)
    lk64 = lk.to(torch.float64).numpy()
    return lk, [synth.query_batch(name, lk, step=s, lk64=lk64) for s in range(steps)]


def bench_retrieve16m(reps=20, inp=None):
    """16,777,216-token resident context (262144 chunks of 64, K/V ~51.5 GB):
    32 query chunks retrieve top-8 from every chunk, then attend and fuse."""
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    name = "retrieve16m"
    cfg = synth.workload(name)
    lk, (qb,) = inp if inp is not None else long_context_inputs(name)
    kd, vd = synth.device_kv(name, "cuda")
    lkd, lqd, qd = lk.cuda(), qb["lq"].cuda(), qb["q"].cuda()
    qpos = qb["q_pos"].cuda()
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    shape = gca.make_shape(G, B, H, Nq, Nk, cfg["S"], cfg["D"], cfg["Dl"], cfg["k"], gca.GCA_BF16,
                           cfg["softmax_one"])
    k = cfg["k"]
    idx = torch.empty((G, B, H, Nq, k), dtype=torch.int32, device="cuda")
    score = torch.empty((G, B, H, Nq, k), device="cuda")
    w = torch.empty_like(score)
    o = torch.empty_like(qd)
    lse = torch.empty((G, B, H, Nq, k, cfg["S"]), device="cuda")
    ws = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)), dtype=torch.uint8,
                     device="cuda")

    def two_calls():
        gca.gca_retrieve(shape, lqd, lkd, qpos, idx, score, w, ws=ws)
        gca.gca_forward(shape, qd, kd, vd, idx, w, o, lse)

    def one_call():  # the slice merge runs inside the forward's kernel
        gca.gca_retrieve_forward(shape, lqd, lkd, qpos, qd, kd, vd, idx, score, w, o, lse, ws=ws)

    for _ in range(3):
        two_calls()
    _, per2 = _timed(two_calls, reps)
    ms2 = _latency(two_calls, reps)
    ref = [t.clone() for t in (idx, score, w, o, lse)]
    for _ in range(3):
        one_call()
    _, per = _timed(one_call, reps)
    ms = _latency(one_call, reps)
    same = all(torch.equal(a, b) for a, b in zip(ref, (idx, score, w, o, lse)))
    scan_ms = per.get("scan_topk", 0.0)
    merge_ms = per2.get("topk_merge", 0.0)
    fwd_ms = per2.get("forward", 0.0)
    mf_ms = per.get("topk_merge_forward", 0.0)
    lk_bytes = G * B * H * Nk * cfg["Dl"] * 2
    scores = G * B * H * Nq * Nk
    best = torch.gather(idx, -1, score.argmax(-1, keepdim=True))[..., 0].cpu()
    hits = float((best == qb["needle"].view(1, 1, 1, Nq)).float().mean())
    del kd, vd
    torch.cuda.empty_cache()
    return {"workload": name, "tokens": Nk * cfg["S"], "query_chunks": Nq, "heads": H,
            "retrieve_fwd_latency_ms": round(ms, 4),
            "call": "gca_retrieve_forward (slice merge inside the forward's kernel)",
            "retrieve_then_forward_latency_ms": round(ms2, 4),
            "one_call_equals_two_calls_bits": bool(same),
            "scan_us": round(scan_ms * 1e3, 2), "merge_forward_us": round(mf_ms * 1e3, 2),
            "merge_us": round(merge_ms * 1e3, 2), "forward_us": round(fwd_ms * 1e3, 2),
            "landmark_scan_GBps": round(lk_bytes / (scan_ms * 1e-3) / 1e9, 1) if scan_ms else None,
            "landmark_scan_roofline_frac": round(lk_bytes / (scan_ms * 1e-3) / HBM_PEAK, 4)
            if scan_ms else None,
            "topk_scores_per_s": round(scores / ((scan_ms + merge_ms) * 1e-3), 1)
            if scan_ms and merge_ms else None,
            "needle_hit_rate": hits, "reps": reps}


def bench_infer1m(steps, inp=None):
    """1,048,576-token resident context (16384 chunks): per chunk step, one new
    query chunk retrieves top-8 of 16383 candidates (with a planted needle),
    attends and fuses.  Latency of each step from HIP events."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    name = "infer1m_step"
    cfg = synth.workload(name)
    lk, batches = inp if inp is not None else long_context_inputs(name, steps)
    kd, vd = synth.device_kv(name, "cuda")
    lkd = lk.cuda()
    G, B, H, Nk, S, k = cfg["G"], cfg["B"], cfg["H"], cfg["n_key"], cfg["S"], cfg["k"]
    qs = torch.stack([b["q"] for b in batches]).cuda()
    lqs = torch.stack([b["lq"] for b in batches]).cuda()
    needles = torch.stack([b["needle"] for b in batches])
    qpos = batches[0]["q_pos"].cuda()
    shape = gca.make_shape(G, B, H, 1, Nk, S, cfg["D"], cfg["Dl"], k, gca.GCA_BF16,
                           cfg["softmax_one"])
    idx = torch.empty((steps, G, B, H, 1, k), dtype=torch.int32, device="cuda")
    score = torch.empty((steps, G, B, H, 1, k), device="cuda")
    w = torch.empty_like(score)
    o = torch.empty_like(qs)
    lse = torch.empty((steps, G, B, H, 1, k, S), device="cuda")
    ws = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)), dtype=torch.uint8,
                     device="cuda")

    def step(s):  # retrieval + forward in one call (the merge inside the forward's kernel)
        gca.gca_retrieve_forward(shape, lqs[s], lkd, qpos, qs[s], kd, vd, idx[s], score[s], w[s],
                                 o[s], lse[s], ws=ws)

    def step_two_calls(s):
        gca.gca_retrieve(shape, lqs[s], lkd, qpos, idx[s], score[s], w[s], ws=ws)
        gca.gca_forward(shape, qs[s], kd, vd, idx[s], w[s], o[s], lse[s])

    def latencies(fn):
        for s in range(10):
            fn(s)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for s in range(steps):
            fn(s)
            ev[s + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]) * 1e3

    lat2 = latencies(step_two_calls)
    lat = latencies(step)
    best = torch.gather(idx, -1, score.argmax(-1, keepdim=True))[..., 0, 0].cpu()
    hits = float((best == needles.view(steps, 1, 1, 1)).float().mean())
    graph = bench_infer1m_graph(shape, lqs, qs, lkd, kd, vd, qpos, ws, idx, o, min(steps, 200))
    del kd, vd
    torch.cuda.empty_cache()
    return {"workload": name, "tokens": Nk * S, "steps": steps,
            "call": "gca_retrieve_forward (slice merge inside the forward's kernel)",
            "step_latency_us_p50": round(float(np.percentile(lat, 50)), 2),
            "step_latency_us_p99": round(float(np.percentile(lat, 99)), 2),
            "step_latency_us_mean": round(float(lat.mean()), 2),
            "two_calls_step_latency_us_p50": round(float(np.percentile(lat2, 50)), 2),
            "needle_hit_rate": hits, "hip_graph": graph}


def bench_infer1m_graph(shape, lqs, qs, lkd, kd, vd, qpos, ws, idx_eager, o_eager, steps,
                        per_graph=10):
    """GPU time of the step without host work in between: per_graph consecutive
    retrieve + forward steps (each on its own query chunk and outputs) captured in one
    HIP graph (torch.cuda.CUDAGraph), so that a replay is one launch from the host and
    the replay time over per_graph is the GPU's latency per step.  The replays' idx and
    O must equal the eager steps' bits (checked on the host)."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as gca
    k, S = shape.top_k, shape.chunk_size
    idx_g = torch.empty_like(idx_eager[:per_graph])
    score_g = torch.empty(idx_g.shape, dtype=torch.float32, device="cuda")
    w_g = torch.empty_like(score_g)
    o_g = torch.empty_like(o_eager[:per_graph])
    lse_g = torch.empty(tuple(idx_g.shape) + (S,), dtype=torch.float32, device="cuda")

    def body():
        for s in range(per_graph):
            gca.gca_retrieve_forward(shape, lqs[s], lkd, qpos, qs[s], kd, vd, idx_g[s], score_g[s],
                                     w_g[s], o_g[s], lse_g[s], ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    exact = True
    for _ in range(3):  # replays checked against the eager steps, synchronised
        idx_g.fill_(-7)
        o_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        exact = exact and torch.equal(idx_g, idx_eager[:per_graph]) and torch.equal(
            o_g, o_eager[:per_graph])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lat = []
    for _ in range(max(1, steps // per_graph)):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1) * 1e3 / per_graph)
    lat = np.array(lat)
    del g
    return {"steps_per_graph": per_graph, "replays": len(lat),
            "gpu_step_latency_us_p50": round(float(np.percentile(lat, 50)), 2),
            "gpu_step_latency_us_p99": round(float(np.percentile(lat, 99)), 2),
            "replays_equal_eager_bits": bool(exact)}


def bench_infer1m_offload(steps, inp=None):
    """The 1M-token inference step with K/V offloaded to pinned host memory:
    landmarks stay in HBM; per step the scan picks 8 chunks per head, only
    those tiles cross the host link (gca_gather_kv), and the forward runs on
    the packed tiles.  Also the device-to-host rate of offloading the whole
    K/V, the transfer the pages size at > 20 GB/s."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth
    name = "infer1m_step"
    cfg = synth.workload(name)
    kd, vd = synth.device_kv(name, "cuda")
    kh = torch.empty(tuple(kd.shape), dtype=kd.dtype, pin_memory=True)
    vh = torch.empty(tuple(vd.shape), dtype=vd.dtype, pin_memory=True)
    kv_bytes = 2 * kd.numel() * kd.element_size()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kh.copy_(kd, non_blocking=True)
    vh.copy_(vd, non_blocking=True)
    torch.cuda.synchronize()
    offload_s = time.perf_counter() - t0
    del kd, vd
    torch.cuda.empty_cache()
    if inp is not None:
        lk, batches = inp
    else:
        lk, batches = long_context_inputs(name, steps)
    lkd = lk.cuda()
    G, B, H, Nk, S, k = cfg["G"], cfg["B"], cfg["H"], cfg["n_key"], cfg["S"], cfg["k"]
    qs = torch.stack([b["q"] for b in batches]).cuda()
    lqs = torch.stack([b["lq"] for b in batches]).cuda()
    needles = torch.stack([b["needle"] for b in batches])
    qpos = batches[0]["q_pos"].cuda()
    shape = gca.make_shape(G, B, H, 1, Nk, S, cfg["D"], cfg["Dl"], k, gca.GCA_BF16,
                           cfg["softmax_one"])
    packed = gca.make_shape(G, B, H, 1, k, S, cfg["D"], cfg["Dl"], k, gca.GCA_BF16,
                            cfg["softmax_one"])
    idx = torch.empty((steps, G, B, H, 1, k), dtype=torch.int32, device="cuda")
    score = torch.empty((steps, G, B, H, 1, k), device="cuda")
    w = torch.empty_like(score)
    o = torch.empty_like(qs)
    lse = torch.empty((steps, G, B, H, 1, k, S), device="cuda")
    kp = torch.empty((G, B, H, k, S, cfg["D"]), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    ip = torch.empty((G, B, H, 1, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)), dtype=torch.uint8,
                     device="cuda")

    def step(s):
        gca.gca_retrieve(shape, lqs[s], lkd, qpos, idx[s], score[s], w[s], ws=ws)
        gca.gca_gather_kv(shape, idx[s], kh, vh, kp, vp, ip)
        gca.gca_forward(packed, qs[s], kp, vp, ip, w[s], o[s], lse[s])

    for s in range(10):
        step(s)
    torch.cuda.synchronize()
    gca.gca_timing_enable(True)
    gca.gca_timing_collect()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for s in range(steps):
        step(s)
        ev[s + 1].record()
    torch.cuda.synchronize()
    gca.gca_timing_enable(False)
    per = {n: v[0] / v[1] for n, v in gca.gca_timing_collect().items() if v[1]}
    lat = np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]) * 1e3
    best = torch.gather(idx, -1, score.argmax(-1, keepdim=True))[..., 0, 0].cpu()
    hits = float((best == needles.view(steps, 1, 1, 1)).float().mean())
    gather_us = per.get("gather_kv", 0.0) * 1e3
    tile_bytes = G * B * H * k * 2 * S * cfg["D"] * 2
    del kh, vh
    return {"workload": name, "kv_location": "pinned host memory", "tokens": Nk * S,
            "steps": steps,
            "step_latency_us_p50": round(float(np.percentile(lat, 50)), 2),
            "step_latency_us_p99": round(float(np.percentile(lat, 99)), 2),
            "gather_us": round(gather_us, 2),
            "kernel_avg_us": {n: round(v * 1e3, 2) for n, v in per.items()},
            "gathered_bytes_per_step": tile_bytes,
            "host_link_gather_GBps": round(tile_bytes / (gather_us * 1e-6) / 1e9, 2)
            if gather_us else None,
            "offload_kv_bytes": kv_bytes,
            "offload_d2h_GBps": round(kv_bytes / offload_s / 1e9, 2),
            "pages_reference": "host link > 20 GB/s: 8 GB offloaded in < 0.4 s",
            "needle_hit_rate": hits}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GCA hot path here runs on a single MI355X "
              "(every (g, b, h) head is independent; see the design notes for sharding)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import retrieval_sparse_attention_amd as gca
    import synth

    # Host inputs of every leg first, then the oracle's worker pool, forked
    # before anything touches the GPU (the workers inherit the inputs).
    cfg = synth.workload(WORKLOAD)
    x = synth.training_inputs(WORKLOAD)
    x_fwd = None if args.no_extras else synth.training_inputs("train16k_fwd", with_dout=False)
    inp16m = inp1m = None
    if not args.no_long_context:
        inp16m = long_context_inputs("retrieve16m")
        inp1m = long_context_inputs("infer1m_step", args.infer_steps)
    pool, workers = None, 0
    if not args.no_cpu_baseline:
        import multiprocessing as mp
        _CPU["train"] = dict(x=x, cfg=cfg)
        if x_fwd is not None:
            _CPU["fwd"] = dict(x=x_fwd, cfg=synth.workload("train16k_fwd"))
        if inp1m is not None:
            c1 = synth.workload("infer1m_step")
            lk1, batches = inp1m
            _CPU["infer1m"] = dict(cfg=c1, lk=lk1, q_pos=c1["q_pos"],
                                   lqs=torch.stack([b["lq"] for b in batches]),
                                   qs=torch.stack([b["q"] for b in batches]),
                                   kpool=_tile_pool(64, 64, 41), vpool=_tile_pool(64, 64, 42))
        if inp16m is not None:
            lk16, (qb16,) = inp16m
            _CPU["retrieve16m"] = dict(cfg=synth.workload("retrieve16m"), lk=lk16,
                                       lq=qb16["lq"], q=qb16["q"], q_pos=qb16["q_pos"],
                                       kpool=_tile_pool(64, 64, 51), vpool=_tile_pool(64, 64, 52))
        workers = cpu_workers()
        pool = mp.get_context("fork").Pool(workers, initializer=_worker_init)
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a ROCm GPU")
    gca.load()
    torch.cuda.set_device(0)
    d = {key: val.contiguous().cuda() for key, val in x.items() if key != "cfg"}
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, k = cfg["S"], cfg["D"], cfg["Dl"], cfg["k"]
    shape = gca.make_shape(G, B, H, Nq, Nk, S, D, Dl, k, gca.GCA_BF16, cfg["softmax_one"],
                           cfg["attn_scale"], cfg["score_scale"])
    dev = "cuda"
    idx = torch.empty((G, B, H, Nq, k), dtype=torch.int32, device=dev)
    score = torch.empty((G, B, H, Nq, k), dtype=torch.float32, device=dev)
    w = torch.empty_like(score)
    o = torch.empty_like(d["q"])
    lse = torch.empty((G, B, H, Nq, k, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    dw, dscore = torch.empty_like(score), torch.empty_like(score)
    dlq = torch.empty(tuple(d["lq"].shape), dtype=torch.float32, device=dev)
    dlk = torch.empty(tuple(d["lk"].shape), dtype=torch.float32, device=dev)
    ws_r = gca.gca_workspace_size(shape, gca.OP_RETRIEVE)
    ws_b = gca.gca_workspace_size(shape, gca.OP_BACKWARD)
    wsr = torch.empty(max(ws_r, 256), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(ws_b, 256), dtype=torch.uint8, device=dev)

    def step():
        gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], idx, score, w, ws=wsr)
        gca.gca_forward(shape, d["q"], d["k"], d["v"], idx, w, o, lse)
        gca.gca_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"],
                         dq, dk, dv, dw, dscore, dlq, dlk, ws=wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    # the headline: K steps with the library's per-kernel event timing off
    gca.gca_timing_enable(False)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps
    # per-kernel times: a second pass of K steps with an event pair around every launch
    gca.gca_timing_enable(True)
    gca.gca_timing_collect()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    gca.gca_timing_enable(False)
    per_kernel = gca.gca_timing_collect()
    step_ms_timed = ev0.elapsed_time(ev1) / args.steps
    tokens = B * Nq * S
    value = tokens / (step_ms / 1e3)
    pairs = int((idx >= 0).sum().item())
    work = kernel_work(cfg, pairs)
    kernels = {}
    for name, (tot, n) in per_kernel.items():
        if n:
            kernels[name] = dict(avg_us=round(tot / n * 1e3, 2), launches=n)
    dom = max(kernels,
              key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    peaks = measure_peaks()
    print(f"[bench] measured peaks: {peaks['hbm_read_GBps']} GB/s read, "
          f"{peaks['copy_read_plus_write_GBps']} GB/s copy, "
          f"{peaks['mfma_bf16_dense_TFLOPs']} TFLOP/s bf16 MFMA, tile gather "
          f"{peaks['gather_l2_GBps']} / {peaks['gather_llc_GBps']} / {peaks['gather_hbm_GBps']} "
          f"GB/s (L2 / last-level cache / HBM)", file=sys.stderr, flush=True)
    roof = with_measured(roofline_entry(dom, kernels[dom]["avg_us"] * 1e-6, work[dom]), peaks)
    sw = step_work(cfg, pairs)
    t_step_roof = max(sw["bytes"] / HBM_PEAK, sw["flops"] / MFMA_BF16_PEAK)
    step_roof = {"bytes": sw["bytes"], "flops": sw["flops"],
                 "bound": "hbm" if sw["bytes"] / HBM_PEAK >= sw["flops"] / MFMA_BF16_PEAK
                 else "mfma",
                 "roofline_us": round(t_step_roof * 1e6, 2),
                 "roofline_tokens_per_s": round(B * Nq * S / t_step_roof, 1),
                 "frac": round(t_step_roof / (step_ms * 1e-3), 4),
                 "frac_of_measured_peaks": round(
                     max(sw["bytes"] / (peaks["hbm_read_GBps"] * 1e9),
                         sw["flops"] / (peaks["mfma_bf16_dense_TFLOPs"] * 1e12))
                     / (step_ms * 1e-3), 4),
                 "note": "whole step (retrieve + forward + backward) against max(HBM, MFMA) "
                         "time of its algorithmic bytes and flops (5 tile products per pair "
                         "in the backward, as the math needs)"}
    digest = source_digest()
    roof["traffic"] = traffic_for(dom, digest)
    roof["algorithmic_bytes"] = work[dom]["bytes"]
    roof["algorithmic_flops"] = work[dom]["flops"]
    for name in kernels:
        if name in work:
            e = with_measured(roofline_entry(name, kernels[name]["avg_us"] * 1e-6, work[name]),
                              peaks)
            kernels[name].update(bound=e["bound"], frac=e["frac"],
                                 frac_of_measured_peak=e["frac_of_measured_peak"])
    gathered = S * D * 2 * 2 * pairs  # K and V (or Q and dO) tiles of every pair
    for name in ("forward", "backward_q", "backward_kv"):
        if name in kernels:
            rate = gathered / (kernels[name]["avg_us"] * 1e-6) / 1e9
            kernels[name].update(gathered_GB=round(gathered / 1e9, 3),
                                 gather_GBps=round(rate, 1),
                                 frac_of_l2_gather_peak=round(rate / peaks["gather_l2_GBps"], 4))
    print(f"[bench] timed {args.steps} steps: {step_ms:.3f} ms/step, dominant {dom}",
          file=sys.stderr, flush=True)
    if args.copy_ref > 0:
        n = args.copy_ref // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy reference: {n} bytes read, {n} bytes written", file=sys.stderr,
              flush=True)
        del src, dst
    swa_res = None
    if not args.no_swa:
        swa_res = bench_swa(args.steps)
        print(f"[bench] sliding-window attention step: {swa_res['ms_per_step']} ms",
              file=sys.stderr, flush=True)
    extra = fwd16k = tiles = None
    if not args.no_extras:
        extra = bench_cold_and_copy(step)
        print(f"[bench] cold step: {extra['cold_ms_per_step_median']} ms", file=sys.stderr,
              flush=True)
        fwd16k = bench_train16k_fwd(args.steps, x_fwd)
        print(f"[bench] 16K forward (one group): {fwd16k['ms_per_step']} ms", file=sys.stderr,
              flush=True)
        tiles = bench_tile_sizes(args.steps)
        print("[bench] other tile sizes: " + ", ".join(f"{kk} {v['ms_per_step']} ms"
                                                       for kk, v in tiles.items()),
              file=sys.stderr, flush=True)
    gumbel = None
    if not args.no_gumbel:
        bufs = (idx, score, w, o, lse, dq, dk, dv, dw, dscore, dlq, dlk, wsr, wsb)
        gumbel = bench_gumbel_step(shape, d, bufs, args.steps)
        gumbel["scan_us_without_noise"] = kernels.get("scan_topk", {}).get("avg_us")
        print(f"[bench] Gumbel top-k training step: {gumbel['ms_per_step']} ms",
              file=sys.stderr, flush=True)
    long_ctx = {}
    if not args.no_long_context:
        long_ctx["retrieve16m"] = bench_retrieve16m(inp=inp16m)
        r16 = long_ctx["retrieve16m"]
        if r16.get("landmark_scan_GBps"):
            r16["landmark_scan_frac_of_measured_read"] = round(
                r16["landmark_scan_GBps"] / peaks["hbm_read_GBps"], 4)
        print(f"[bench] 16M retrieval: {long_ctx['retrieve16m']['retrieve_fwd_latency_ms']} ms",
              file=sys.stderr, flush=True)
        long_ctx["infer1m_step"] = bench_infer1m(args.infer_steps, inp1m)
        print(f"[bench] 1M inference step p50: "
              f"{long_ctx['infer1m_step']['step_latency_us_p50']} us", file=sys.stderr, flush=True)
        long_ctx["infer1m_step_offloaded_kv"] = bench_infer1m_offload(args.infer_steps, inp1m)
        print(f"[bench] 1M inference step, K/V in host memory, p50: "
              f"{long_ctx['infer1m_step_offloaded_kv']['step_latency_us_p50']} us",
              file=sys.stderr, flush=True)
    cpu = None
    if pool is not None:
        print(f"[bench] CPU baseline: the oracle on {workers} worker processes",
              file=sys.stderr, flush=True)
        base = cpu_baselines(pool, workers)
        pool.close()
        pool.join()
        cpu = base.get("train")
        if fwd16k is not None and "fwd" in base:
            fwd16k["cpu_baseline"] = base["fwd"]
        if "infer1m" in base:
            long_ctx["infer1m_step"]["cpu_baseline"] = base["infer1m"]
        if "retrieve16m" in base:
            long_ctx["retrieve16m"]["cpu_baseline"] = base["retrieve16m"]
    line = {
        "metric": "GCA fwd+bwd tokens/s @16K ctx k=8",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/8 q,k,v,landmarks; N(0,1) dO)",
        "config": {"workload": WORKLOAD, "G": G, "B": B, "H": H, "tokens": Nq * S,
                   "chunk_size": S, "head_dim": D, "landmark_dim": Dl, "top_k": k,
                   "softmax_one": cfg["softmax_one"], "pairs": pairs,
                   "step": "gca_retrieve + gca_forward + gca_backward"},
        "roofline": roof,
        "step_roofline": step_roof,
        "measured_peaks": peaks,
        "ms_per_step_with_kernel_events": round(step_ms_timed, 4),
        "cpu_baseline": cpu,
        "kernels": kernels,
        "long_context": long_ctx or None,
        "cold_and_copy": extra,
        "train16k_fwd": fwd16k,
        "tile_sizes": tiles,
        "gumbel_train_step": gumbel,
        "sliding_window_step": swa_res,
        "wall_s_timed": round(wall, 3),
        "source_digest": digest,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
