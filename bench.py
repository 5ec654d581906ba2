#!/usr/bin/env python3
"""HHR decode benchmark on one MI355X: append + decode of one Llama-3.1-8B-shaped layer at 128K.

Workload (synthetic, seeded): 32 query heads, 8 KV heads, d = 128, bf16 K/V, batch 1, context
131072 tokens, pages of 16, 128-bit codes, page keep ratio 1/16, token budget 4096; keys
N(0,1) with 4 outlier channels x10 per KV head and 32 planted high-logit keys per query head;
one new token appended per step (the index is updated), then the decode step runs.

A "step" is hhr_append_decode (append one token, then decode) on one layer. The benchmark
cycles over --layers distinct layer instances (separate K/V, index and sequence state in HBM) so
the ~256 MB Infinity Cache cannot serve a step from the previous visit. Three passes, each W
warm-up steps then exactly K timed steps bracketed by torch.cuda.synchronize():
  1. launches with HIP start/stop events that the runtime records around each of the five
     kernels' own execution: per-kernel durations and the roofline figure (events_us_per_step);
  2. plain launches on one stream, no events: the headline us/step/layer;
  3. replay of one captured HIP graph per layer instance (graph_us_per_step; on this stack a
     graph replay of the five kernels is slower than the plain launches).

Prints ONE JSON line. Options: --gpus (must be 1), --steps, --warmup, --layers,
--no-cpu-baseline, --quiet, --copy-calibration (a 512 MiB device copy only, to scale the HBM
byte counters of rocprofv3).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CTX = 131072
HBM_PEAK_GBS = 8000.0
KERNELS = ("prep", "page_bound", "select", "sparse_attn", "combine")


def log(msg, quiet):
    if not quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, L):
    """Bytes each kernel must move per launch (one layer, one append + decode step) at context L.

    prep:       q, k_new, v_new, R and W read; q~ and the query codes written; the appended
                token's K and V rows and code written, its page's extrema column pair read and
                written.
    page_bound: min+max of every page of every KV head (128 ch x 8 B per page), q~ read, U
                written (4 B per query head and page).
    select:     U and the query code read, the codes of the kept pages' tokens (16 B per
                candidate and query head), the selected indices written.
    sparse_attn: K and V rows of the selected tokens (2 x 256 B per token and query head),
                indices and q read, one (o, m, l) partial per 256 tokens written.
    combine:    the partials read, the output written.
    """
    d, S, nb = cfg.head_dim, cfg.page_size, cfg.hash_bits
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    P = -(-L // S)
    n_keep = min(P, max(1, math.ceil(cfg.keep_ratio * P)))
    k = min(cfg.token_budget, n_keep * S)
    esz = 2
    return {
        "prep": Hq * d * esz + Hkv * 2 * d * esz + Hkv * d * d * 4 + Hkv * d * nb * 4
                + Hq * d * 4 + Hq * nb // 8
                + Hkv * 2 * d * esz + Hkv * nb // 8 + Hkv * 2 * d * 4 * 2,
        "page_bound": Hkv * P * d * 8 + Hq * d * 4 + Hq * P * 4,
        "select": Hq * P * 4 + Hq * nb // 8 + Hq * n_keep * S * (nb // 8) + Hq * k * 4,
        "sparse_attn": Hq * k * 2 * d * esz + Hq * k * 4 + Hq * d * esz
        + Hq * -(-k // 256) * (d + 2) * 4,
        "combine": Hq * -(-k // 256) * (d + 2) * 4 + Hq * d * 4,
    }


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_decode_gkr_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, digest):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except ValueError:
        return None
    if t.get("source_digest") != digest:
        return None
    v = t.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")
    return float(v) if v is not None else None


def time_builder(hb, cache, R, W, cfg, L, quiet, reps=5):
    """Index build of the whole 128K layer (MFMA path for bf16 keys), timed with HIP events.
    Rebuilding is idempotent, so the same cache is rebuilt `reps` times after one warm-up."""
    stream = hb.current_stream()
    ev = hb.HipEvents(2)
    hb.build_pages(cache, R, W)
    ms = []
    for _ in range(reps):
        ev.record(0, stream)
        hb.build_pages(cache, R, W)
        ev.record(1, stream)
        import torch
        torch.cuda.synchronize()
        ms.append(ev.elapsed_ms(0, 1))
    ev.close()
    t = sorted(ms)[len(ms) // 2] * 1e-3
    d, nb, Hkv = cfg.head_dim, cfg.hash_bits, cfg.num_kv_heads
    useful = 2.0 * L * Hkv * d * (d + nb)            # K x [R | W]
    executed = 2.0 * L * Hkv * d * (3 * d + 2 * nb)  # bf16 pieces: 3 of R, 2 of W
    log(f"builder: {t * 1e6:.1f} us for {L} tokens x {Hkv} KV heads", quiet)
    return {"us": round(t * 1e6, 1), "tokens": L * Hkv, "useful_TFLOPs": round(useful / t / 1e12, 2),
            "mfma_TFLOPs": round(executed / t / 1e12, 2), "mfma_peak_TFLOPs": 2500.0,
            "mfma_frac": round(executed / t / 1e12 / 2500.0, 4), "dtype": "bf16 MFMA, fp32 acc"}


def cpu_baseline(cfg, data, quiet, budget_s=10.0):
    """The oracle, as it stands, on a bounded sample: one KV group (KV head 0 and its 4 query
    heads) of the same layer: one append then the 4 heads' decode, repeated for ~budget_s.
    The per-step time of the whole layer is that sample's time x Hkv (the groups are
    independent and identical in cost)."""
    import numpy as np
    from oracle import hhr_oracle as orc
    from long_context_decode_gkr_amd import synth
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    S, G = cfg.page_size, cfg.group
    L0 = int(data["seq_lens"][0])
    K, V = data["K"][0, 0], data["V"][0, 0]
    R, W = data["R"][0], data["W"][0]
    log("cpu baseline: oracle index of KV head 0 (untimed setup)", quiet)
    lo, hi, kc = orc.build_head(K, L0, R, W, S)
    Lmax = K.shape[0]
    Pmax = Lmax // S
    st0 = dict(lo=np.zeros((Pmax, 128), np.float32), hi=np.zeros((Pmax, 128), np.float32),
               codes=np.zeros((Lmax, cfg.hash_bits // 32), np.uint32))
    st0["lo"][:len(lo)], st0["hi"][:len(hi)], st0["codes"][:L0] = lo, hi, kc
    kn, vn = synth.append_tokens(cfg, 1)
    scale = orc.default_scale(128)
    Kc, Vc = K.copy(), V.copy()
    reps, spent = 0, 0.0
    while spent < budget_s and reps < 1000:
        st = dict(K=Kc, V=Vc, lo=st0["lo"].copy(), hi=st0["hi"].copy(), codes=st0["codes"], L=L0)
        t = time.perf_counter()
        orc.append_head(st, kn[0, 0, 0], vn[0, 0, 0], R, W, S)
        for h in range(G):
            orc.decode_head(data["q"][0, h], st["K"], st["V"], st["L"], st["lo"], st["hi"],
                            st["codes"], R, W, S, cfg.keep_ratio, cfg.token_budget, scale)
        spent += time.perf_counter() - t
        reps += 1
    us_layer = spent / reps * cfg.num_kv_heads * 1e6
    return {"value": round(us_layer, 1), "unit": "us/step/layer", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"KV head 0 and its {G} query heads of the same 128K layer (append + "
                       f"decode), {reps} repetitions in {spent:.1f} s, scaled by "
                       f"{cfg.num_kv_heads} KV groups; index build untimed")}


def copy_calibration(mib=512, reps=3):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters: each launch reads and writes exactly `mib` MiB."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 512 MiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the HHR decode path has no multi-GPU mode "
              "(it would shard by KV head with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from long_context_decode_gkr_amd import binding as hb
    from long_context_decode_gkr_amd import synth

    q = args.quiet
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hb.load()
    cfg = synth.CONFIGS[3]
    NL, K, Wm = args.layers, args.steps, args.warmup
    visits = -(-(3 * (K + Wm)) // NL)     # appends per layer over the three passes
    L0 = CTX - visits                      # every layer ends at <= 128K tokens
    log(f"generating the 128K layer (L0={L0})", q)
    t0 = time.time()
    data = synth.make_layer(cfg, max_seq_len=CTX, lens=[L0])
    log(f"  {time.time() - t0:.1f} s", q)
    dims = hb.make_dims(1, 32, 8, 16, 128, CTX, kv_dtype=hb.HHR_BF16)
    dev = torch.device("cuda")
    bf = torch.bfloat16
    qd = torch.from_numpy(data["q"]).to(dev).to(bf)
    Rd = torch.from_numpy(data["R"]).to(dev)
    Wd = torch.from_numpy(data["W"]).to(dev)
    layers = []
    first = hb.Cache(dims)
    first.K.copy_(torch.from_numpy(data["K"]).to(dev).to(bf))
    first.V.copy_(torch.from_numpy(data["V"]).to(dev).to(bf))
    first.seq_lens.fill_(L0)
    hb.build_pages(first, Rd, Wd)
    torch.cuda.synchronize()
    builder = time_builder(hb, first, Rd, Wd, cfg, L0, q)
    layers.append(first)
    for _ in range(NL - 1):
        c = hb.Cache(dims)
        for name in ("K", "V", "page_min", "page_max", "codes", "seq_lens", "append_ticket"):
            getattr(c, name).copy_(getattr(first, name))
        layers.append(c)
    kn, vn = synth.append_tokens(cfg, visits)
    knd = torch.from_numpy(kn).to(dev).to(bf)
    vnd = torch.from_numpy(vn).to(dev).to(bf)
    dec = hb.Decoder(dims, cfg.keep_ratio, cfg.token_budget)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev)
    cache_structs = [c.struct() for c in layers]
    P = dict(q=qd.data_ptr(), R=Rd.data_ptr(), W=Wd.data_ptr(), ws=dec.ws.data_ptr(),
             out=out.data_ptr())

    def step(i, dbg, stream, visit=None):
        li = i % NL
        v = i // NL if visit is None else visit
        hb.hhr_append_decode(dims, dec.params, cache_structs[li], knd[v].data_ptr(),
                             vnd[v].data_ptr(), P["q"], P["R"], P["W"], P["ws"], dec.ws_bytes,
                             P["out"], dbg, stream)

    # ---- pass 1 (launches with events): per-kernel durations from HIP events that the runtime
    # records around each kernel's own execution on the decode stream (hipExtLaunchKernel)
    stream = hb.current_stream()
    NE = 2 * len(KERNELS)
    ev = hb.HipEvents(NE * K)
    dbgs = [hb.DebugStruct(None, None, None, None, None, None, None, None, ev.address(NE * i))
            for i in range(K)]
    log(f"events pass: warm-up {Wm}, timed {K} steps over {NL} layer instances", q)
    for i in range(Wm):
        step(i, None, stream)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(Wm + i, dbgs[i], stream)
    torch.cuda.synchronize()
    events_ms = (time.perf_counter() - t_start) * 1e3 / K
    # events [NE i + 2 j] and [NE i + 2 j + 1]: start and stop of kernel j of step i
    per = {n: [ev.elapsed_ms(NE * i + 2 * j, NE * i + 2 * j + 1) for i in range(K)]
           for j, n in enumerate(KERNELS)}
    ev.close()

    # ---- pass 2 (plain launches on one stream): the headline figure
    log(f"stream pass: warm-up {Wm}, timed {K} steps", q)
    base = Wm + K
    for i in range(Wm):
        step(base + i, None, stream)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(base + Wm + i, None, stream)
    torch.cuda.synchronize()
    stream_ms = (time.perf_counter() - t_start) * 1e3 / K

    # ---- pass 3 (graph replay): one captured step per layer instance
    graphs = []
    gstream = torch.cuda.Stream()
    with torch.cuda.stream(gstream):
        for li in range(NL):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=gstream):
                step(li, None, hb.current_stream(), visit=(li % visits))
            graphs.append(gr)
    torch.cuda.synchronize()
    log(f"graph pass: warm-up {Wm}, timed {K} steps", q)
    for i in range(Wm):
        graphs[i % NL].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        graphs[(Wm + i) % NL].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t_start) * 1e3 / K
    ms_step = stream_ms
    avg_ms = {n: float(np.mean(v)) for n, v in per.items()}
    Lavg = L0 + visits // 2
    alg = algorithmic_bytes(cfg, Lavg)
    kern = {}
    for n in KERNELS:
        kern[n] = {"avg_us": round(avg_ms[n] * 1e3, 2), "p50_us": round(float(np.median(per[n])) * 1e3, 2),
                   "alg_bytes": alg[n],
                   "alg_GBps": round(alg[n] / (avg_ms[n] * 1e-3) / 1e9, 1)}
    dominant = max(("page_bound", "sparse_attn"), key=lambda n: avg_ms[n])
    digest = kernel_source_digest()
    traffic = load_traffic(dominant, digest)
    achieved = alg[dominant] / (avg_ms[dominant] * 1e-3) / 1e9
    step_bytes = sum(alg.values())
    us = ms_step * 1e3
    result = {
        "metric": "HHR decode us/step/layer at 128K ctx (32q/8kv, d128) + % HBM roofline",
        "value": round(us, 2),
        "unit": "us/step/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 5),
        "events_us_per_step": round(events_ms * 1e3, 2),
        "graph_us_per_step": round(graph_ms * 1e3, 2),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) keys with outlier channels and planted keys; "
                "random orthogonal R, Gaussian W)",
        "config": {"workload": "Llama-3.1-8B-shaped layer, 128K context, append+decode",
                   "batch": 1, "seq_len": CTX, "q_heads": 32, "kv_heads": 8, "head_dim": 128,
                   "kv_dtype": "bf16", "page_size": 16, "hash_bits": 128, "keep_ratio": 1 / 16,
                   "token_budget": 4096, "layers_cycled": NL, "context_range": [L0, CTX]},
        "keys_scored_per_s": round(cfg.num_q_heads * Lavg / (ms_step * 1e-3), 1),
        "step_alg_bytes": step_bytes,
        "step_hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernels": kern,
        "builder": builder,
        "kernel_source_digest": digest,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, data, q)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
