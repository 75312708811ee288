"""Decode-attention throughput of the LLA hot path on one MI355X.

One step = what one generated token costs every sequence in the store:
D*T decode-attention calls in loop-major order (for t: for layer), each
reading that layer's whole latent slab for all B sequences, then D encode
appends writing the new token's latents (slot N-1, overwritten in steady
state).  Inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line (rank 0, N = 1 GPU):
  value      = B / step time  (tokens/s, all sequences)
  roofline   = per-head stores (HBM-bound): algorithmic bytes of one decode
               call / its average duration, against 8 TB/s;
               LLA-2D stores (bound by the matrix cores): the K-side
               contraction's flops / the call's duration, against 2.5 PFLOP/s
               dense bf16.  Durations are HIP events recorded on the launch
               stream around every call of the timed region.
               traffic = HBM bytes per launch from the committed rocprofv3
               FETCH_SIZE / WRITE_SIZE summary (null if the kernel changed).
  cpu_baseline = the fp64 oracle timed on a bounded sample on host cores

--path fast / final_loop time the two uncompressed-cache paths on the same
workload instead (a cache [B, D, L, N, H, 2, d]): the serving fast path
(every loop's K/V reconstructed once into the cache, L = T, plain
flash-decode; each step encodes the new token and reconstructs its T loops)
and the final-loop control (L = 1: every loop's query attends the last
loop's K/V; each step appends the new token's final-loop K/V).  When the
cache does not fit in HBM the line says so (value null) instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LLA decode-attn tokens/s at B=768, 4k ctx, ρ=21.3 + % of HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# Names of the decode split kernels whose counters the traffic summary reads
# (the same expression goes to rocprofv3 --kernel-include-regex); the split-K
# encode kernel is not one of them.
SPLIT_KERNELS = r"decode\w*_split|kv_split"
# (r_k, r_v) pairs of the multi-query store pass (d = 128, at most 16 queries)
MQ_RANKS = {(16, 32), (32, 64), (48, 80)}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
CSRC = os.path.join(ROOT, "looped_transformer_decode_amd", "csrc")
# FETCH_SIZE / WRITE_SIZE of a plain 8 GB device copy (one dispatch) read 3,906,278 KiB
# and 7,812,500 KiB: the fetch counter reports half of the bytes read.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="extreme_batch_b768_ctx4k")
    ap.add_argument("--path", choices=("lla", "fast", "final_loop"), default="lla",
                    help="lla: the latent store (default); fast: reconstructed full K/V cache; "
                         "final_loop: the final-loop-reuse control")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences (0 = the workload's own batch)")
    ap.add_argument("--svd-init", action="store_true",
                    help="time the SVD codec initialisation of one layer's codecs (K and V, all "
                         "heads) on synthetic calibration trajectories of the workload's shape")
    ap.add_argument("--n-cal", type=int, default=4096, help="calibration rows for --svd-init")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle timing sample (0 disables it)")
    ap.add_argument("--splits", type=int, default=0,
                    help="context splits per decode call (0 = the library's choice)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GB",
                    help="instead of the benchmark, copy a buffer of this size a few times "
                         "(reference for HBM byte counters)")
    ap.add_argument("--write-ceiling", type=float, default=0.0, metavar="GB",
                    help="instead of the decode step: time a plain streaming write and a plain "
                         "copy of a buffer of this size (the ceilings of the write-bound kernels)")
    ap.add_argument("--read-ceiling", type=float, default=0.0, metavar="GB",
                    help="instead of the benchmark, time a plain streaming-read kernel over a "
                         "buffer of this size (the practical HBM read ceiling)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the benchmark, time a register-only bf16 MFMA kernel "
                         "(the practical matrix-core ceiling)")
    ap.add_argument("--no-encode", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--inflight", action="store_true",
                    help="decode with the step's n_new tokens in flight (multi-query causal "
                         "call with their exact loop-t keys and values)")
    ap.add_argument("--eager", action="store_true",
                    help="report the eagerly launched step time (no HIP graph replay)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "output directories (FETCH_SIZE, WRITE_SIZE) and exit")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, pos_plus_one: int) -> int:
    """Bytes one decode call must move: the latent slab slots 0..pos of
    every sequence, the queries and outputs, and W_up,t / mu_t."""
    store = w.B * pos_plus_one * w.store_heads * w.R * w.elt_bytes
    q_out = 2 * w.B * w.H * w.d * 4
    rows = w.H * w.d
    codec = rows * w.R * w.elt_bytes + 2 * rows * 4
    return store + q_out + codec


def kv_algorithmic_bytes(w, pos_plus_one: int) -> int:
    """Bytes one flash-decode call over an uncompressed cache must move: the
    K and V rows of slots 0..pos of every head and sequence, q and out."""
    return w.B * pos_plus_one * w.H * 2 * w.d * w.elt_bytes + 2 * w.B * w.H * w.d * 4


def kernel_source(w, path="lla") -> str:
    """Source of the split kernel whose counters a traffic summary holds;
    path: lla, inflight (multi-query store pass), fast or final_loop."""
    if path in ("fast", "final_loop"):
        return os.path.join(CSRC, "kvcache.hip")
    if path == "inflight":
        return os.path.join(CSRC, "decode_mq.hip")
    return os.path.join(CSRC, "decode2d_mfma.hip" if w.variant == "2d" else "decode_mfma.hip")


def inflight_bytes(w, nq: int) -> int:
    """Bytes of one in-flight call: the store slots before pos0 once, plus
    q, k_new, v_new and out of every query, W_up,t and mu_t."""
    return (algorithmic_bytes(w, w.N - w.n_new) - 2 * w.B * w.H * w.d * 4
            + 4 * w.B * nq * w.H * w.d * 4)


def encode_bytes(w) -> int:
    """Bytes one encode-append call must move: x of both axes, W_down and mu
    of both axes, the latents written and the start positions."""
    K = w.T * w.width
    rows = w.B * w.n_new * w.store_heads
    return (2 * rows * K * w.elt_bytes + w.store_heads * K * w.R * w.elt_bytes
            + 2 * w.store_heads * K * 4 + rows * w.R * w.elt_bytes + 4 * w.B)


def traffic_file(w, path="lla") -> str:
    tag = "" if path == "lla" else f"{path}_"
    return os.path.join(ROOT, "profiles", f"traffic_{tag}{w.name}.json")


def kernel_sha(w, path="lla") -> str:
    return hashlib.sha256(open(kernel_source(w, path), "rb").read()).hexdigest()


def traffic_for_current_kernel(w, path="lla"):
    """HBM bytes per launch of the decode split kernel from the committed
    rocprofv3 counter summary, or None when absent, taken on a different
    kernel source or at another batch."""
    try:
        with open(traffic_file(w, path)) as f:
            t = json.load(f)
        if t.get("kernel_sha256") != kernel_sha(w, path) or t.get("batch", w.B) != w.B:
            return None
        return t.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def algorithmic_flops(w, pos_plus_one: int) -> int:
    """Matrix-core work of one LLA-2D decode call: the K-side contraction
    (tokens x d x r_k per head) that reconstruction, RoPE and q.k share."""
    return 2 * w.B * pos_plus_one * w.H * w.d * w.r_k


def summarize_counters(w, fetch_dir: str, write_dir: str, path: str = "lla") -> dict:
    """Per-launch HBM bytes of the decode split kernel from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), scaled by
    the copy-kernel calibration; written to profiles/traffic_<workload>.json."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and re.search(SPLIT_KERNELS, r["Kernel_Name"]):
                    vals.append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit(f"no {counter} rows for a split kernel under {d}")
        return sum(vals) / len(vals), len(vals)

    fetch, nf = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, nw = per_dispatch(write_dir, "WRITE_SIZE")
    hbm = fetch * 1024 * FETCH_SCALE + write * 1024 * WRITE_SCALE
    algo = (algorithmic_bytes(w, w.N) if path == "lla" else
            inflight_bytes(w, w.n_new) if path == "inflight" else kv_algorithmic_bytes(w, w.N))
    res = {"workload": w.name, "path": path, "batch": w.B,
           "kernel_source": os.path.relpath(kernel_source(w, path), ROOT),
           "kernel_sha256": kernel_sha(w, path), "fetch_kib_per_dispatch": round(fetch, 1),
           "write_kib_per_dispatch": round(write, 1), "dispatches": [nf, nw],
           "fetch_scale": FETCH_SCALE, "write_scale": WRITE_SCALE,
           "hbm_bytes_per_launch": int(hbm), "algorithmic_bytes_per_launch": algo}
    with open(traffic_file(w, path), "w") as f:
        json.dump(res, f, indent=1)
    return res


def host_cpu() -> dict:
    """The host cores this process may run on and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def cpu_baseline(w, codec, budget_s: float):
    """Oracle decode of the (layer 0, loop 0) call, one sequence at a time
    until the time budget is spent; scaled to tokens/s of the whole step."""
    from oracle import lla_oracle as O
    from synth.workloads import store_slab
    layer, t = 0, 0
    q = codec.q(layer, t, 4)
    wk, wv = codec.w_up("k", layer, t), codec.w_up("v", layer, t)
    mk = O.loop_slice(codec.mu("k", layer), t, w.width)
    mv = O.loop_slice(codec.mu("v", layer), t, w.width)
    done, spent = 0, 0.0
    while spent < budget_s and done < w.B:
        b = done % 4
        slab = store_slab(w, b, layer)
        t0 = time.perf_counter()
        if w.variant == "2d":
            O.decode_2d(slab[:, 0, :w.r_k], slab[:, 0, w.r_k:], q[b], wk[0], wv[0], mk[0], mv[0],
                        w.N - 1)
        else:
            O.decode(slab[..., :w.r_k], slab[..., w.r_k:], q[b], wk, wv, mk, mv, w.N - 1)
        spent += time.perf_counter() - t0
        done += 1
    per_seq = spent / done
    t_step = per_seq * w.B * w.D * w.T
    return {"value": w.B / t_step, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "t_call_s": per_seq * w.B, **host_cpu(),
            "sample": f"{done} sequence(s) x {w.H} heads of the (layer 0, loop 0) call at pos "
                      f"{w.N - 1}, {spent:.1f} s; scaled x{w.B}/{done} sequences x "
                      f"{w.D * w.T} calls per step"}


def memory_summary(bytes_total: int, batch: int, hbm_bytes: int) -> dict:
    """Footprint of the cache or store and how many sequences of this
    shape fit in the GPU's memory."""
    per_seq = bytes_total // batch
    return {"bytes": bytes_total, "per_sequence_bytes": per_seq, "hbm_bytes": hbm_bytes,
            "max_batch_in_hbm": int(hbm_bytes // per_seq)}


def cpu_baseline_kv(w, budget_s: float):
    """Oracle flash-decode (decode_cache) of one (layer, loop) call, one
    sequence at a time on seeded slabs of the cache's shape, until the time
    budget is spent; scaled to tokens/s of the whole step."""
    from oracle import lla_oracle as O
    from synth import gen
    calls = w.D * w.T
    done, spent = 0, 0.0
    while spent < budget_s and done < w.B:
        slab = gen.normal(w.seed, 7000 + done % 4, (w.N, w.H, 2, w.d))
        q = gen.normal(w.seed, 7100 + done % 4, (w.H, w.d))
        t0 = time.perf_counter()
        for h in range(w.H):
            O.decode_cache(slab[:, h, 0], slab[:, h, 1], q[h], w.N - 1)
        spent += time.perf_counter() - t0
        done += 1
    t_step = spent / done * w.B * calls
    return {"value": w.B / t_step, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "t_call_s": spent / done * w.B, **host_cpu(),
            "sample": f"{done} sequence(s) x {w.H} heads of one flash-decode call at pos "
                      f"{w.N - 1}, {spent:.1f} s; scaled x{w.B}/{done} sequences x {calls} "
                      f"calls per step"}


def run_svd_init(args, w, torch, L, dev):
    """SVD initialisation of one layer's codecs (every head, K then V axis)
    from n_cal synthetic calibration rows per codec: rank-8 loop trajectories
    plus N(0, 0.05^2) noise, the long-recurrence recipe.  Reports codecs per
    second and the fp32 matrix-core work per second (the GEMMs run on
    v_mfma_f32_32x32x2_f32) against MI355X's 157.3 TFLOP/s fp32 matrix peak."""
    from synth import gen
    G, K, n = w.store_heads, w.T * w.width, args.n_cal
    log(f"[bench] svd init: workload {w.name}, {G} codecs per axis, K={K}, n_cal={n}, "
        f"r_k={w.r_k}, r_v={w.r_v}")
    x = np.stack([gen.low_rank_trajectory(w.seed, 9000 + g, n, K) for g in range(G)], axis=1)
    xd = torch.from_numpy(gen.f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).to(dev)
    xd = xd.view(torch.bfloat16) if w.dtype == "bf16" else xd.view(torch.bfloat16).float()
    tdt = xd.dtype
    outs = {}
    for r in (w.r_k, w.r_v):
        outs[r] = (torch.empty((G, K), dtype=torch.float32, device=dev),
                   torch.empty((G, K, r), dtype=tdt, device=dev),
                   torch.empty((w.T, G, w.width, r), dtype=tdt, device=dev),
                   torch.empty((G, r), dtype=torch.float32, device=dev),
                   torch.empty(L.lla_svd_init_workspace_bytes(G, w.T, w.width, r),
                               dtype=torch.uint8, device=dev))

    def step(timer=None):
        for r in (w.r_k, w.r_v):
            mu, wd, wu, sg, ws = outs[r]
            if timer is not None:
                timer.start(torch.cuda.current_stream())
            L.lla_svd_init(xd, w.T, w.width, r, mu, wd, wu, sg, ws)
            if timer is not None:
                timer.stop(torch.cuda.current_stream())

    args.eager = True
    ms_eager, ms_step, call_ms = time_step(args, step, torch.cuda.current_stream(), torch, 2)
    # matrix-core work per call: the centred Gram matrix (its 128 x 128 tiles
    # on and above the diagonal), then per iteration C Q and two CholeskyQR
    # passes, then the Rayleigh-Ritz products (fp32 GEMMs)
    iters = 16
    flops = {}
    tiles = (K + 127) // 128
    for r in (w.r_k, w.r_v):
        m = min(r + 16, 128, K)
        gram = 2 * n * 128 * 128 * tiles * (tiles + 1) // 2
        orth = 2 * (2 * K * m * m + 2 * K * m * m)          # two CholeskyQR passes
        flops[r] = G * (gram + (iters + 1) * (2 * K * K * m + orth) + 2 * K * m * m
                        + 2 * K * m * r)
    total_flops = sum(flops.values())
    achieved = total_flops / (ms_step / 1e3) / 1e12
    # error of the codec on its calibration rows (Eckart-Young: discarded energy)
    xc = xd.float() - xd.float().mean(0, keepdim=True)
    energy = (xc * xc).sum(dim=(0, 2)).double()
    # Eckart-Young: with the leading singular values of the larger-rank call,
    # the error of every smaller rank is the energy beyond its first r values
    rmax = max(w.r_k, w.r_v)
    sg2 = outs[rmax][3].double() ** 2
    err = {}
    for r in sorted({1, 2, 4, 6, 7, 8, 9, 10, 12, 16, 24, 32, 48, 64, 80, w.r_k, w.r_v}):
        if r <= rmax:
            err[str(r)] = float(((energy - sg2[:, :r].sum(1)) / energy).mean())
    peak = 157.3
    res = {"metric": "SVD codec initialisation: codecs/s (one layer's K and V codecs of every head)",
           "value": round(2 * G / (ms_step / 1e3), 2), "unit": "codecs/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": w.name, "codecs_per_axis": G, "K": K, "n_cal": n,
                      "ranks": [w.r_k, w.r_v], "iterations": iters,
                      "input": "rank-8 loop trajectories + N(0, 0.05^2), " + w.dtype},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                        "kernel": "all lla_svd_init kernels (fp32 matrix-core GEMMs; the fp64 "
                                  "Cholesky and Jacobi steps are latency-bound)",
                        "flops_per_step": total_flops,
                        "call_ms": [round(float(v), 3) for v in call_ms[:2]]},
           "calibration_error_vs_r": err, "cpu_baseline": None}
    print(json.dumps(res), flush=True)


def run_kv_path(args, w, torch, L, dev):
    """The serving fast path or the final-loop control on workload w."""
    from synth import gen
    from synth.device import fill_hash_normal
    from synth.workloads import TID_Q, TID_X_K, TID_X_V, Codec, store_key

    fast = args.path == "fast"
    metric = ("fast-path decode tokens/s (latents reconstructed into a full K/V cache, "
              "flash-decode)" if fast else
              "final-loop-control decode tokens/s (last loop's K/V cached, reused by every loop)")
    cache = L.KvCache(w.dtype, batch=w.B, layers=w.D, loops=w.T if fast else 1, max_ctx=w.N,
                      heads=w.H, d_head=w.d)
    sdesc = L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                          d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v)
    cache_bytes = L.lla_kv_cache_bytes(cache)
    need = cache_bytes + (L.lla_store_bytes(sdesc) if fast else 0)
    free, hbm = torch.cuda.mem_get_info(dev)
    config = {"workload": w.name, "path": args.path, "variant": w.variant, "B": w.B,
              "layers": w.D, "ctx": w.N, "heads": w.H, "d_head": w.d, "loops": w.T,
              "cache_loops": cache.loops, "calls_per_step": w.D * w.T}
    res = {"metric": metric, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
           "data": "synthetic", "config": config,
           "memory": memory_summary(cache_bytes, w.B, hbm)}
    log(f"[bench] {args.path} path, workload {w.name} B={w.B}: cache {cache_bytes / 1e9:.2f} GB "
        f"(+ latent store {L.lla_store_bytes(sdesc) / 1e9:.2f} GB)" if fast else
        f"[bench] {args.path} path, workload {w.name} B={w.B}: cache {cache_bytes / 1e9:.2f} GB")
    if need > free - (4 << 30):
        log(f"[bench] does not fit: {need / 1e9:.1f} GB needed, {free / 1e9:.1f} GB free")
        res.update({"value": None, "ms_per_step": None, "roofline": None, "cpu_baseline": None,
                    "oom": {"bytes_needed": need, "bytes_free": free}})
        print(json.dumps(res), flush=True)
        return

    cache.tensor = torch.empty(cache.shape, dtype=cache.torch_dtype, device=dev)
    rope = L.lla_kv_rope_table_fill(cache).to(dev)
    tdt = cache.torch_dtype
    is2d = w.variant == "2d"
    q = torch.empty((w.D, w.T, w.B, w.H, w.d), dtype=torch.float32, device=dev)
    fill_hash_normal(q, gen.stream_key(w.seed, TID_Q))
    pos = torch.full((w.B,), w.N - 1, dtype=torch.int32, device=dev)
    start = torch.full((w.B,), w.N - w.n_new, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    ws = L.kv_workspace(cache, args.splits)
    stream = torch.cuda.current_stream()

    def up(x, dtype):
        x32 = np.asarray(x, np.float32)
        if dtype == torch.float32:
            return torch.from_numpy(x32).to(dev)
        return torch.from_numpy(gen.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(tdt)

    fill_stats = None
    if fast:
        store = L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N,
                              heads=w.H, d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v,
                              device=dev)
        fill_hash_normal(store.tensor, store_key(w))
        codec = Codec(w)
        wk, wv, mk, mv, wdk, wdv, muk, muv = {}, {}, {}, {}, [], [], [], []
        for l in range(w.D):
            for t in range(w.T):
                a, b_ = codec.w_up("k", l, t), codec.w_up("v", l, t)
                wk[l, t] = up(a.reshape(-1, w.r_k) if is2d else a, tdt)
                wv[l, t] = up(b_.reshape(-1, w.r_v) if is2d else b_, tdt)
                m1 = codec.mu("k", l)[:, t * w.width:(t + 1) * w.width]
                m2 = codec.mu("v", l)[:, t * w.width:(t + 1) * w.width]
                mk[l, t] = up(m1.reshape(-1) if is2d else m1, torch.float32)
                mv[l, t] = up(m2.reshape(-1) if is2d else m2, torch.float32)
            wdk.append(up(codec.w_down("k", l)[0] if is2d else codec.w_down("k", l), tdt))
            wdv.append(up(codec.w_down("v", l)[0] if is2d else codec.w_down("v", l), tdt))
            muk.append(up(codec.mu("k", l)[0] if is2d else codec.mu("k", l), torch.float32))
            muv.append(up(codec.mu("v", l)[0] if is2d else codec.mu("v", l), torch.float32))
        K = w.T * w.width
        xshape = (w.D, w.B, w.n_new, K) if is2d else (w.D, w.B, w.n_new, w.H, K)
        xk = torch.empty(xshape, dtype=tdt, device=dev)
        xv = torch.empty(xshape, dtype=tdt, device=dev)
        fill_hash_normal(xk, gen.stream_key(w.seed, TID_X_K))
        fill_hash_normal(xv, gen.stream_key(w.seed, TID_X_V))
        encode = L.lla2d_encode_append if is2d else L.lla_encode_append
        # prefill: every layer's and loop's K/V reconstructed from the latents once
        torch.cuda.synchronize()
        fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fe[0].record(stream)
        for l in range(w.D):
            for t in range(w.T):
                L.lla_kv_fill_from_store(store, l, wk[l, t], wv[l, t], mk[l, t], mv[l, t], 0, w.N,
                                         rope, cache, t)
        fe[1].record(stream)
        torch.cuda.synchronize()
        fill_ms = fe[0].elapsed_time(fe[1]) / (w.D * w.T)
        per_fill = cache_bytes // (w.D * w.T)
        lat_read = L.lla_store_bytes(store) // w.D
        fill_stats = {"kernel": "kv_fill_mfma (one lla_kv_fill_from_store call, all slots)",
                      "launch_us": round(fill_ms * 1e3, 2), "bytes_written": per_fill,
                      "bytes_read": lat_read,
                      "GBps": round((per_fill + lat_read) / (fill_ms / 1e3) / 1e9, 1)}
        log(f"[bench] reconstruct-to-cache: {fill_ms * 1e3:.1f} us per (layer, loop) fill, "
            f"{fill_stats['GBps']} GB/s")
    else:
        fill_hash_normal(cache.tensor, gen.stream_key(w.seed, 50))
        kv_new = torch.empty((2, w.D, w.B, w.n_new, w.H, w.d), dtype=torch.float32, device=dev)
        fill_hash_normal(kv_new, gen.stream_key(w.seed, 51))
    torch.cuda.synchronize()
    log(f"[bench] splits={args.splits or L.lla_kv_decode_auto_splits(cache)}")

    def step(timer=None):
        for t in range(w.T):
            for l in range(w.D):
                if timer is not None:
                    timer.start(stream)
                L.lla_kv_decode_attn(cache, l, t if fast else 0, q[l, t], pos, rope, out, ws,
                                     n_splits=args.splits)
                if timer is not None:
                    timer.stop(stream)
        for l in range(w.D):
            if fast:
                encode(store, l, xk[l], xv[l], muk[l], muv[l], wdk[l], wdv[l], start)
                for t in range(w.T):
                    L.lla_kv_fill_from_store(store, l, wk[l, t], wv[l, t], mk[l, t], mv[l, t],
                                             w.N - w.n_new, w.n_new, rope, cache, t)
            else:
                L.lla_kv_append(cache, l, 0, kv_new[0, l], kv_new[1, l], start, rope)

    ms_eager, ms_step, call_ms = time_step(args, step, stream, torch, w.D * w.T)
    bytes_call = kv_algorithmic_bytes(w, w.N)
    achieved = bytes_call / (call_ms.mean() / 1e3) / 1e9
    res.update({
        "value": round(w.B / (ms_step / 1e3), 2), "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "launch": "eager" if args.eager else "hip_graph_replay",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for_current_kernel(w, args.path),
                     "kernel": "kv_split (+ kv_merge) (one lla_kv_decode_attn call)",
                     "bytes_per_launch": bytes_call,
                     "launch_us": round(call_ms.mean() * 1e3, 2)}})
    config["splits"] = args.splits or L.lla_kv_decode_auto_splits(cache)
    if fill_stats:
        res["reconstruct_to_cache"] = fill_stats
    res["cpu_baseline"] = cpu_baseline_kv(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(res), flush=True)


class CallTimer:
    """HIP events around every decode call of a pass, created up front (the
    first creation of a timing event can stall the host for milliseconds)."""

    def __init__(self, torch, n: int):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        self.i = 0

    def start(self, stream):
        self.ev[self.i][0].record(stream)

    def stop(self, stream):
        self.ev[self.i][1].record(stream)
        self.i += 1

    def ms(self):
        return np.array([a.elapsed_time(b) for a, b in self.ev[:self.i]])


def time_step(args, step, stream, torch, calls_per_step: int, enc_per_step: int = 0):
    """Warm-up; a plain eager pass (ms/step as launched from the host); a
    pass with events around every decode call, queued behind a spin kernel
    so that the GPU never waits for the host inside it (the events then
    bracket the kernels alone); then, unless --eager, the step captured as a
    HIP graph and replayed.  Returns (eager ms/step, reported ms/step,
    per-call ms array), plus the per-call ms of the encode appends when
    enc_per_step > 0 (step then takes a second timer for them)."""
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    def timed(run):
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for _ in range(args.steps):
            run()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    ms_eager = timed(step)
    timer = CallTimer(torch, calls_per_step * args.steps)
    etimer = CallTimer(torch, enc_per_step * args.steps) if enc_per_step else None
    torch.cuda.synchronize()
    try:  # hold the queue for longer than the host needs to enqueue the pass
        torch.cuda._sleep(int(3e6 * (2.0 * ms_eager * args.steps + 20.0)))
    except (AttributeError, RuntimeError):
        pass
    for _ in range(args.steps):
        if etimer is None:
            step(timer)
        else:
            step(timer, etimer)
    torch.cuda.synchronize()
    call_ms = timer.ms()
    log(f"[bench] {args.steps} eager steps: {ms_eager:.3f} ms/step; decode call mean "
        f"{call_ms.mean() * 1e3:.1f} us (min {call_ms.min() * 1e3:.1f}, "
        f"max {call_ms.max() * 1e3:.1f})")
    ms_step = ms_eager
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        ms_step = timed(graph.replay)
        log(f"[bench] {args.steps} graph replays: {ms_step:.3f} ms/step")
    if etimer is not None:
        return ms_eager, ms_step, call_ms, etimer.ms()
    return ms_eager, ms_step, call_ms


def run_read_ceiling(args, torch):
    """A plain streaming read of a buffer larger than the caches (the
    practical HBM read ceiling the decode kernels are compared with):
    workgroups of 256 threads, each walking one contiguous range with eight
    16-byte nontemporal loads per thread in flight."""
    from synth.device import read_stream
    dev = torch.device("cuda:0")
    n = int(args.read_ceiling * 1e9) // (16 * 2048) * (16 * 2048)
    src = torch.zeros(n // 4, dtype=torch.int32, device=dev)
    results = {}
    for blocks in (2048, 4096, 8192):
        sink = torch.empty(blocks * 256 * 4, dtype=torch.int32, device=dev)
        for _ in range(3):
            read_stream(src, sink, blocks)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        reps = max(args.steps, 5)
        ev[0].record()
        for _ in range(reps):
            read_stream(src, sink, blocks)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        results[blocks] = (ms, n / (ms / 1e3) / 1e9)
        log(f"[bench] read ceiling: {blocks} workgroups, {n / 1e9:.2f} GB in {ms * 1e3:.1f} us: "
            f"{results[blocks][1]:.1f} GB/s")
    best = max(results, key=lambda b: results[b][1])
    print(json.dumps({"metric": "streaming-read GB/s (plain read kernel, context for the decode "
                                "kernels' HBM fraction)",
                      "value": round(results[best][1], 1), "unit": "GB/s",
                      "peak": HBM_PEAK_GBS, "frac": round(results[best][1] / HBM_PEAK_GBS, 4),
                      "bytes": n, "kernel": "read_stream (synth/fill.hip)",
                      "workgroups": best,
                      "sweep": {str(b): {"launch_us": round(v[0] * 1e3, 2),
                                         "GBps": round(v[1], 1)} for b, v in results.items()}}),
          flush=True)


def run_write_ceiling(args, torch):
    """A plain streaming write, and a plain copy, of a buffer larger than the
    caches: workgroups of 256 threads taking 32 KB chunks in turn (those in
    flight neighbours in memory), eight 16-byte stores per thread in flight.
    The copy's bytes count its reads and its writes."""
    from synth.device import write_stream
    dev = torch.device("cuda:0")
    n = int(args.write_ceiling * 1e9) // (16 * 2048) * (16 * 2048)
    dst = torch.empty(n // 4, dtype=torch.int32, device=dev)
    src = torch.zeros(n // 4, dtype=torch.int32, device=dev)
    out = {}
    for mode, s_arg, nbytes in (("write", None, n), ("copy", src, 2 * n)):
        results = {}
        for blocks in (2048, 8192, 32768):
            for _ in range(3):
                write_stream(dst, blocks, s_arg)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            reps = max(args.steps, 5)
            ev[0].record()
            for _ in range(reps):
                write_stream(dst, blocks, s_arg)
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / reps
            results[blocks] = (ms, nbytes / (ms / 1e3) / 1e9)
            log(f"[bench] {mode} ceiling: {blocks} workgroups, {nbytes / 1e9:.2f} GB in "
                f"{ms * 1e3:.1f} us: {results[blocks][1]:.1f} GB/s")
        best = max(results, key=lambda b: results[b][1])
        # torch's own fill and copy kernels of the same buffers, beside it
        lib_fn = (lambda: dst.fill_(7)) if s_arg is None else (lambda: dst.copy_(src))
        for _ in range(3):
            lib_fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        reps = max(args.steps, 5)
        ev[0].record()
        for _ in range(reps):
            lib_fn()
        ev[1].record()
        torch.cuda.synchronize()
        lib_ms = ev[0].elapsed_time(ev[1]) / reps
        lib_gbs = nbytes / (lib_ms / 1e3) / 1e9
        log(f"[bench] {mode} ceiling: torch {'fill_' if s_arg is None else 'copy_'} "
            f"{lib_ms * 1e3:.1f} us: {lib_gbs:.1f} GB/s")
        top = max(results[best][1], lib_gbs)
        out[mode] = {"GBps": round(top, 1), "frac": round(top / HBM_PEAK_GBS, 4),
                     "kernel": "write_stream" if results[best][1] >= lib_gbs else
                               ("torch fill_" if s_arg is None else "torch copy_"),
                     "write_stream": {"workgroups": best, "GBps": round(results[best][1], 1)},
                     "torch": {"launch_us": round(lib_ms * 1e3, 2), "GBps": round(lib_gbs, 1)},
                     "sweep": {str(b): {"launch_us": round(v[0] * 1e3, 2), "GBps": round(v[1], 1)}
                               for b, v in results.items()}}
    print(json.dumps({"metric": "streaming-write GB/s (best plain write: write_stream of "
                                "synth/fill.hip or torch fill_; the plain copy beside it, reads "
                                "plus writes), context for the write-bound kernels",
                      "value": out["write"]["GBps"], "unit": "GB/s", "peak": HBM_PEAK_GBS,
                      "frac": out["write"]["frac"], "bytes": n, "write": out["write"],
                      "copy": out["copy"]}), flush=True)


def run_mfma_ceiling(args, torch):
    """Register-only v_mfma_f32_32x32x16_bf16 chains (four independent
    accumulators per wave) at one to four waves per SIMD: the bf16
    matrix-core throughput this box sustains, against the 2.5 PFLOP/s
    nominal peak."""
    from synth.device import mfma_spin
    dev = torch.device("cuda:0")
    iters = 4096
    results = {}
    for waves_per_simd in (1, 2, 4):
        blocks = 256 * waves_per_simd            # 4 waves per workgroup: one per SIMD
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        mfma_spin(blocks, 64, sink)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        mfma_spin(blocks, iters, sink)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        flops = blocks * 4 * 4 * iters * 32768
        results[waves_per_simd] = (ms, flops / (ms / 1e3) / 1e12)
        log(f"[bench] mfma ceiling: {waves_per_simd} wave(s)/SIMD, {ms * 1e3:.1f} us: "
            f"{results[waves_per_simd][1]:.1f} TFLOP/s")
    best = max(results, key=lambda k: results[k][1])
    # How far the matrix cores and the vector ALU of one SIMD overlap: one
    # MFMA-only and one FMA-only wave per SIMD, each alone and together.
    from synth.device import mfma_valu_overlap
    blocks, it = 256, 8192
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    ovl = {}
    for mode, name in ((1, "mfma_only"), (2, "valu_only"), (3, "both")):
        mfma_valu_overlap(blocks, 64, mode, sink)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        mfma_valu_overlap(blocks, it, mode, sink)
        ev[1].record()
        torch.cuda.synchronize()
        ovl[name] = round(ev[0].elapsed_time(ev[1]) * 1e3, 1)
    ovl["hidden_share_of_shorter"] = round(
        (ovl["mfma_only"] + ovl["valu_only"] - ovl["both"]) / min(ovl["mfma_only"], ovl["valu_only"]), 3)
    log(f"[bench] mfma/valu overlap (us): {ovl}")
    print(json.dumps({"metric": "bf16 MFMA TFLOP/s (register-only 32x32x16 chains, context for "
                                "the LLA-2D roofline fraction)",
                      "value": round(results[best][1], 1), "unit": "TFLOP/s",
                      "peak": MFMA_BF16_PEAK_TFLOPS,
                      "frac": round(results[best][1] / MFMA_BF16_PEAK_TFLOPS, 4),
                      "kernel": "mfma_spin (synth/fill.hip)", "waves_per_simd": best,
                      "sweep": {str(k): {"us": round(v[0] * 1e3, 1), "TFLOPs": round(v[1], 1)}
                                for k, v in results.items()},
                      "mfma_valu_overlap_us": ovl}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path here (the hot path "
              "would shard by sequence with no exchange).", file=sys.stderr)
        sys.exit(2)

    if args.summarize_counters:
        from synth.workloads import WORKLOADS
        w = WORKLOADS[args.workload]
        if args.batch:
            w = w.scaled(B=args.batch)
        tag = "inflight" if args.inflight else args.path
        print(json.dumps(summarize_counters(w, *args.summarize_counters, tag)))
        return

    import torch

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 1e9) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": ms,
                          "GBps_read_plus_write": 2 * n * 4 / ms / 1e6}), flush=True)
        return

    if args.read_ceiling > 0:
        run_read_ceiling(args, torch)
        return
    if args.write_ceiling > 0:
        run_write_ceiling(args, torch)
        return
    if args.mfma_ceiling:
        run_mfma_ceiling(args, torch)
        return

    import looped_transformer_decode_amd as L
    from synth import gen
    from synth.device import fill_hash_normal
    from synth.workloads import TID_Q, TID_X_K, TID_X_V, WORKLOADS, Codec, store_key

    w = WORKLOADS[args.workload]
    if args.batch:
        w = w.scaled(B=args.batch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.svd_init:
        run_svd_init(args, w, torch, L, dev)
        return
    if args.path != "lla":
        run_kv_path(args, w, torch, L, dev)
        return
    log(f"[bench] workload {w.name}: B={w.B} D={w.D} N={w.N} H={w.H} d={w.d} T={w.T} "
        f"r_k={w.r_k} r_v={w.r_v} {w.variant} {w.dtype}; store {w.store_bytes / 1e9:.2f} GB")

    store = L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                          d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v, device=dev)
    t0 = time.time()
    fill_hash_normal(store.tensor, store_key(w))
    torch.cuda.synchronize()
    log(f"[bench] store filled in {time.time() - t0:.1f} s")
    rope = L.rope_table(store, dev)
    codec = Codec(w)
    tdt = store.torch_dtype
    is2d = w.variant == "2d"
    width = w.width

    def up(x, dtype):
        x32 = np.asarray(x, np.float32)
        if dtype == torch.float32:
            return torch.from_numpy(x32).to(dev)
        return torch.from_numpy(gen.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(tdt)

    # codec tensors of every (layer, loop)
    wk, wv, mk, mv = {}, {}, {}, {}
    wdk, wdv, muk, muv = [], [], [], []
    for l in range(w.D):
        for t in range(w.T):
            a, b_ = codec.w_up("k", l, t), codec.w_up("v", l, t)
            wk[l, t] = up(a.reshape(-1, w.r_k) if is2d else a, tdt)
            wv[l, t] = up(b_.reshape(-1, w.r_v) if is2d else b_, tdt)
            m1 = codec.mu("k", l)[:, t * width:(t + 1) * width]   # mu_t: loop-t block
            m2 = codec.mu("v", l)[:, t * width:(t + 1) * width]
            mk[l, t] = up(m1.reshape(-1) if is2d else m1, torch.float32)
            mv[l, t] = up(m2.reshape(-1) if is2d else m2, torch.float32)
        wdk.append(up(codec.w_down("k", l)[0] if is2d else codec.w_down("k", l), tdt))
        wdv.append(up(codec.w_down("v", l)[0] if is2d else codec.w_down("v", l), tdt))
        muk.append(up(codec.mu("k", l)[0] if is2d else codec.mu("k", l), torch.float32))
        muv.append(up(codec.mu("v", l)[0] if is2d else codec.mu("v", l), torch.float32))
    q = torch.empty((w.D, w.T, w.B, w.H, w.d), dtype=torch.float32, device=dev)
    fill_hash_normal(q, gen.stream_key(w.seed, TID_Q))
    K = w.T * width
    xshape = (w.D, w.B, w.n_new, K) if is2d else (w.D, w.B, w.n_new, w.H, K)
    xk = torch.empty(xshape, dtype=tdt, device=dev)
    xv = torch.empty(xshape, dtype=tdt, device=dev)
    fill_hash_normal(xk, gen.stream_key(w.seed, TID_X_K))
    fill_hash_normal(xv, gen.stream_key(w.seed, TID_X_V))
    pos = torch.full((w.B,), w.N - 1, dtype=torch.int32, device=dev)
    start = torch.full((w.B,), w.N - w.n_new, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    ws = L.workspace(store, args.splits)
    nq = w.n_new if args.inflight else 1
    if args.inflight:
        # the step's n_new tokens run their loops before their latents exist:
        # every decode call is the multi-query call with them in flight
        qi = torch.empty((w.D, w.T, w.B, nq, w.H, w.d), dtype=torch.float32, device=dev)
        fill_hash_normal(qi, gen.stream_key(w.seed, TID_Q) + 1)
        kvi = torch.empty((2, w.D, w.T, w.B, nq, w.H, w.d), dtype=torch.float32, device=dev)
        fill_hash_normal(kvi, gen.stream_key(w.seed, TID_Q) + 2)
        pos0 = start
        out = torch.empty((w.B, nq, w.H, w.d), dtype=torch.float32, device=dev)
        ws = L.workspace(store, args.splits, n_q=nq)
    decode = L.lla2d_decode_attn if is2d else L.lla_decode_attn
    encode = L.lla2d_encode_append if is2d else L.lla_encode_append
    stream = torch.cuda.current_stream()
    log(f"[bench] path={L.lla_decode_path(store)} "
        f"splits={args.splits or L.lla_decode_auto_splits(store)}")

    def step(timer=None, etimer=None):
        for t in range(w.T):
            for l in range(w.D):
                if timer is not None:
                    timer.start(stream)
                if args.inflight:
                    L.lla_decode_attn_inflight(store, l, t, qi[l, t], kvi[0, l, t], kvi[1, l, t],
                                               wk[l, t], wv[l, t], mk[l, t], mv[l, t], pos0,
                                               rope, out, ws, n_splits=args.splits)
                else:
                    decode(store, l, t, q[l, t], wk[l, t], wv[l, t], mk[l, t], mv[l, t], pos,
                           rope, out, ws, n_splits=args.splits)
                if timer is not None:
                    timer.stop(stream)
        if not args.no_encode:
            for l in range(w.D):
                if etimer is not None:
                    etimer.start(stream)
                encode(store, l, xk[l], xv[l], muk[l], muv[l], wdk[l], wdv[l], start)
                if etimer is not None:
                    etimer.stop(stream)

    if args.no_encode:
        ms_eager, ms_step, call_ms = time_step(args, step, stream, torch, w.D * w.T)
        enc_ms = None
    else:
        ms_eager, ms_step, call_ms, enc_ms = time_step(args, step, stream, torch, w.D * w.T, w.D)
    value = w.B * nq / (ms_step / 1e3)   # generated tokens per second, all sequences
    bytes_call = algorithmic_bytes(w, w.N)
    if args.inflight:
        bytes_call = inflight_bytes(w, nq)
    path = L.lla_decode_path(store)
    tag = "inflight" if args.inflight else "lla"
    if w.variant == "2d":
        flops_call = algorithmic_flops(w, w.N)
        achieved = flops_call / (call_ms.mean() / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": traffic_for_current_kernel(w),
                    "kernel": "decode2d_split + decode_merge_batched (one lla2d_decode_attn call)",
                    "flops_per_launch": flops_call, "bytes_per_launch": bytes_call,
                    "hbm_GBps": round(bytes_call / (call_ms.mean() / 1e3) / 1e9, 1),
                    "launch_us": round(call_ms.mean() * 1e3, 2)}
    else:
        achieved = bytes_call / (call_ms.mean() / 1e3) / 1e9
        splits = args.splits or L.lla_decode_auto_splits(store)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic_for_current_kernel(w, tag),
                    "kernel": (("decode_mq_split" if path == "mfma" and 1 < nq <= 16 and w.d == 128
                                and w.variant == "per_head" and (w.r_k, w.r_v) in MQ_RANKS
                                else "decode split kernel")
                               + " + decode_merge_inflight (one lla_decode_attn_inflight call)")
                              if args.inflight else
                              (("decode_mfma_split" if path == "mfma" else "decode_valu_split")
                               + " (one lla_decode_attn call"
                               + (")" if splits == 1 and path == "mfma" else " + decode_merge)")),
                    "bytes_per_launch": bytes_call, "launch_us": round(call_ms.mean() * 1e3, 2)}
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "launch": "eager" if args.eager else "hip_graph_replay",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "variant": w.variant, "B": w.B, "layers": w.D,
                   "ctx": w.N, "heads": w.H, "d_head": w.d, "loops": w.T, "r_k": w.r_k,
                   "r_v": w.r_v, "rho": str(L.lla_compression_ratio(store)),
                   "calls_per_step": w.D * w.T, "encode_appends_per_step": 0 if args.no_encode
                   else w.D, "tokens_per_sequence_per_step": nq,
                   "in_flight": bool(args.inflight),
                   "splits": args.splits or L.lla_decode_auto_splits(store),
                   "path": path},
        "roofline": roofline,
        "memory": memory_summary(L.lla_store_bytes(store), w.B,
                                 torch.cuda.mem_get_info(dev)[1]),
    }
    if enc_ms is not None and len(enc_ms):
        eb = encode_bytes(w)
        ea = eb / (enc_ms.mean() / 1e3) / 1e9
        res["encode"] = {"bound": "hbm", "achieved": round(ea, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ea / HBM_PEAK_GBS, 4),
                         "kernel": f"{'lla2d' if is2d else 'lla'}_encode_append: "
                                   f"{w.B * w.n_new} tokens x {w.store_heads} codecs, "
                                   f"K = {w.T * w.width}",
                         "bytes_per_launch": eb, "launch_us": round(enc_ms.mean() * 1e3, 2),
                         "calls_per_step": w.D}
    if args.cpu_seconds > 0:
        del store, q, xk, xv
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(w, codec, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
