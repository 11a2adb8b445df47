"""Benchmark of the mixed-precision KV transfer path on one MI355X.

One step = the whole path over one request of the Mistral-7B-shaped workload
(32 layers, 32 query / 8 KV heads, head dim 128, 8192 tokens, S = 4 sinks,
3-tier, b = 0.5): per layer the two score passes (row log-sum-exp, then the
MFMA column sums accumulated into the score), tier assignment, pack, dense
unpack and paged unpack (16-token blocks, seeded permuted block table).
Inputs are seeded synthetic tensors, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the fp16-equivalent KV throughput of
pack + dense unpack, 2 * KV_fp16_bytes / (t_pack + t_unpack), from HIP events
recorded on the launch stream inside the timed steps; the score's TFLOP/s and
every stage's time are reported beside it.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mistral7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-score-shapes", action="store_true",
                    help="skip timing the score passes on one Qwen- and one Gemma-shaped layer")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough budget of the oracle's timed sample")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the transfer path is built and timed on a "
              "single MI355X (multi-GPU sharding is a design note, not a measured path).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import serving_sk_score_amd as sk
    from workloads import gen, get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sk.lib()  # fails loudly if the HIP library is not built

    cfg = get_config(args.workload)
    L, Hq, Hkv, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    dev = torch.device("cuda", 0)
    log(f"workload {cfg.name}: L={L} Hq={Hq} Hkv={Hkv} d={d} n={n}; generating inputs")
    t0 = time.time()
    from concurrent.futures import ThreadPoolExecutor

    Q = torch.empty((L, n, Hq, d), dtype=torch.float16, device=dev)
    K = torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev)
    V = torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev)

    def layer_inputs(layer):
        k = gen.keys(cfg, layer)
        return gen.queries(cfg, layer, k=k), k, gen.values(cfg, layer)

    with ThreadPoolExecutor(16) as ex:
        for layer, (q, k, v) in enumerate(ex.map(layer_inputs, range(L))):
            Q[layer].copy_(torch.from_numpy(q))
            K[layer].copy_(torch.from_numpy(k))
            V[layer].copy_(torch.from_numpy(v))
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f} s")

    shape = sk.Shape(L, Hq, Hkv, d)
    shape1 = sk.Shape(1, Hq, Hkv, d)
    pol = sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget)
    plan = sk.plan_make(shape, pol)
    lse = torch.empty((Hq, n), dtype=torch.float32, device=dev)
    cws = torch.empty(max(1, sk.colsum_workspace_bytes(shape1, n)), dtype=torch.uint8, device=dev)
    score = torch.empty(n, dtype=torch.float32, device=dev)
    amap = torch.empty(n, dtype=torch.int32, device=dev)
    order = torch.empty(n, dtype=torch.int32, device=dev)
    payload = torch.empty(plan.payload_bytes, dtype=torch.uint8, device=dev)
    Ko = torch.empty_like(K)
    Vo = torch.empty_like(V)
    bs = 16
    nblk = (n + bs - 1) // bs
    perm = np.random.default_rng(0).permutation(nblk).astype(np.int32)
    block_table = torch.from_numpy(perm).to(dev)
    Kc = torch.empty((L, nblk, bs, Hkv, d), dtype=torch.float16, device=dev)
    Vc = torch.empty_like(Kc)

    # practical bandwidth ceiling (and the counter calibration kernel of the
    # traffic measurement): a device-to-device copy of the K+V bytes
    src = K.view(-1).view(torch.uint8)
    dst = torch.empty_like(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    c0.record()
    for _ in range(3):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 3 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst

    stages = ["rowlse", "colsum", "assign", "pack", "unpack", "unpack_paged"]
    ev = None
    # pack and unpack are timed cold: a 1 GiB write before each of them
    # evicts the 256 MB Infinity Cache (outside their events)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def evict():
        scratch.fill_(0x5A)

    def mark(name, i):
        if ev is not None:
            ev[name][i].record()

    def step():
        for layer in range(L):
            mark("rowlse", 2 * layer)
            sk.score_rowlse(shape1, Q[layer], K[layer], lse)
            mark("rowlse", 2 * layer + 1)
            mark("colsum", 2 * layer)
            sk.score_colsum(shape1, Q[layer], K[layer], lse, score, layer > 0, cws)
            mark("colsum", 2 * layer + 1)
        mark("assign", 0)
        sk.assign_tiers(pol, plan, score, amap, order)
        mark("assign", 1)
        evict()
        mark("pack", 0)
        sk.pack(shape, plan, K, V, amap, order, payload)
        mark("pack", 1)
        evict()
        mark("unpack", 0)
        sk.unpack(shape, plan, payload, amap, Ko, Vo)
        mark("unpack", 1)
        evict()
        mark("unpack_paged", 0)
        sk.unpack_paged(shape, plan, payload, amap, Kc, Vc, block_table, bs)
        mark("unpack_paged", 1)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    nev = {"rowlse": 2 * L, "colsum": 2 * L}
    all_ev = [{s: [torch.cuda.Event(enable_timing=True) for _ in range(nev.get(s, 2))]
               for s in stages} for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    wall0 = time.time()
    start.record()
    for i in range(args.steps):
        ev = all_ev[i]
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps

    # the score variants of the same request, timed on their own (they replace
    # or reweight the score; they are not part of the step)
    def timed(fn, reps):
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    alt = torch.empty(n, dtype=torch.float32, device=dev)
    reps = max(3, args.steps)
    t_kvnorm = timed(lambda: sk.score_kvnorm(shape, K, alt), reps) * 1e-3
    t_recency = timed(lambda: sk.recency_weight(score, 1e-3, alt), reps) * 1e-3

    # cold-tier upgrade of n/8 seeded tokens: fp16 gather, then the paged scatter
    n_up = n // 8
    up_tokens = torch.from_numpy(
        np.random.default_rng(1).choice(n, size=n_up, replace=False).astype(np.int32)).to(dev)
    up_payload = torch.empty(sk.upgrade_bytes(shape, n_up), dtype=torch.uint8, device=dev)
    t_up_pack = timed(lambda: sk.upgrade_pack(shape, K, V, up_tokens, up_payload), reps) * 1e-3
    t_up_paged = timed(lambda: sk.upgrade_unpack_paged(shape, n, up_payload, up_tokens, Kc, Vc,
                                                       block_table, bs), reps) * 1e-3
    up_bytes = 2 * up_payload.numel() + 4 * n_up                 # rows read + written, list

    # decode attention straight from the payload, all layers in one launch
    # (one decode query per layer), and the same kernel over an all-fp16
    # payload of the same request: the bytes a dense-KV attention reads
    qdec = torch.from_numpy((np.random.default_rng(2).standard_normal((L, Hq, d)) * 0.5)
                            .astype(np.float16)).to(dev)
    odec = torch.empty((L, Hq, d), dtype=torch.float32, device=dev)
    ldec = torch.empty((L, Hq), dtype=torch.float32, device=dev)
    dws = torch.empty(max(1, sk.decode_workspace_bytes(shape, plan, L)), dtype=torch.uint8,
                      device=dev)
    t_dec = timed(lambda: sk.decode_attention(shape, plan, payload, qdec, odec, ldec, ws=dws),
                  reps) * 1e-3
    pol16 = sk.Policy(n, cfg.sinks, cfg.three_tier, 1.0)
    plan16 = sk.plan_make(shape, pol16)
    amap16 = torch.empty_like(amap)
    order16 = torch.empty_like(order)
    sk.assign_tiers(pol16, plan16, score, amap16, order16)
    payload16 = torch.empty(plan16.payload_bytes, dtype=torch.uint8, device=dev)
    sk.pack(shape, plan16, K, V, amap16, order16, payload16)
    dws16 = torch.empty(max(1, sk.decode_workspace_bytes(shape, plan16, L)), dtype=torch.uint8,
                        device=dev)
    t_dec16 = timed(lambda: sk.decode_attention(shape, plan16, payload16, qdec, odec, ldec,
                                                ws=dws16), reps) * 1e-3
    del payload16
    dec_io = L * Hq * d * (2 + 4) + L * Hq * 4                    # q in, out and lse written
    dec_bytes = plan.payload_bytes + dec_io
    dec16_bytes = plan16.payload_bytes + dec_io

    # the score passes on one layer of each long-context workload's shape
    # (seeded inputs of that workload): parity cases, not bench lines, timed
    # here so the line shows the passes at their other head counts and d
    score_shapes = {}
    if not args.no_score_shapes:
        for other in ("qwen25_7b_2tier", "gemma2_9b"):
            oc = get_config(other)
            ok_ = gen.keys(oc, 0)
            oq = torch.from_numpy(gen.queries(oc, 0, k=ok_)).to(dev)
            ok_ = torch.from_numpy(ok_).to(dev)
            osh = sk.Shape(1, oc.q_heads, oc.kv_heads, oc.head_dim)
            on = oc.tokens
            olse = torch.empty((oc.q_heads, on), dtype=torch.float32, device=dev)
            osc = torch.empty(on, dtype=torch.float32, device=dev)
            ows = torch.empty(max(1, sk.colsum_workspace_bytes(osh, on)), dtype=torch.uint8,
                              device=dev)
            t_r = timed(lambda: sk.score_rowlse(osh, oq, ok_, olse), 3)
            t_c = timed(lambda: sk.score_colsum(osh, oq, ok_, olse, osc, False, ows), 3)
            f = oc.q_heads * oc.head_dim * on * (on + 1)
            names = score_kernel_names(oc.q_heads, oc.kv_heads, oc.head_dim)
            score_shapes[other] = {
                "layer": f"Hq={oc.q_heads} Hkv={oc.kv_heads} d={oc.head_dim} n={on}",
                "rowlse": {"kernel": names["rowlse"], "ms": round(t_r, 4),
                           "tflops": round(f / (t_r * 1e-3) / 1e12, 1),
                           "frac": round(f / (t_r * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
                "colsum": {"kernel": names["colsum"], "ms": round(t_c, 4),
                           "tflops": round(f / (t_c * 1e-3) / 1e12, 1),
                           "frac": round(f / (t_c * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}}
            del oq, ok_, olse, osc, ows
            log(f"score passes on one {other} layer: {t_r:.3f} + {t_c:.3f} ms")

    # per stage: [steps][launches] durations in ms
    t = {s: np.array([[e[s][2 * j].elapsed_time(e[s][2 * j + 1]) for j in range(len(e[s]) // 2)]
                      for e in all_ev]) for s in stages}
    mean_launch = {s: float(t[s].mean()) for s in stages}          # ms per launch
    per_step_ms = {s: float(t[s].sum(axis=1).mean()) for s in stages}
    step_ms = {s: t[s].sum(axis=1) for s in stages}                # per timed step

    kv_bytes = 2 * L * n * Hkv * d * 2
    pack_bytes = kv_bytes + 4 * n + plan.payload_bytes                  # read K,V + map, write P
    unpack_bytes = plan.payload_bytes + 4 * n + kv_bytes
    t_pack = per_step_ms["pack"] * 1e-3
    t_unpack = per_step_ms["unpack"] * 1e-3
    t_paged = per_step_ms["unpack_paged"] * 1e-3
    value = 2 * kv_bytes / (t_pack + t_unpack) / 1e9
    pass_flops = Hq * d * n * (n + 1)                                   # one pass, one layer
    score_s = (per_step_ms["rowlse"] + per_step_ms["colsum"]) * 1e-3
    score_tflops = 2 * pass_flops * L / score_s / 1e12

    dom = "colsum" if mean_launch["colsum"] >= mean_launch["rowlse"] else "rowlse"
    ach = pass_flops / (mean_launch[dom] * 1e-3) / 1e12
    kernel_name = score_kernel_names(Hq, Hkv, d)[dom]
    nb = pack_batch(Hkv, d)

    def rl(bytes_, sec, kernel):
        gbs = bytes_ / sec / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": bytes_,
                "traffic": counted_traffic(kernel, cfg.name)}

    def call_rl(bytes_, sec):
        gbs = bytes_ / sec / 1e9
        return {"bound": "hbm", "call": "sk_decode_attention", "achieved": round(gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "bytes_per_call": bytes_}

    line = {
        "metric": "KV pack+unpack GB/s (fp16-equiv, % HBM peak); importance-score TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: L={L} Hq={Hq} Hkv={Hkv} d={d} n={n} S={cfg.sinks} "
                               f"b={cfg.budget} {'3' if cfg.three_tier else '2'}-tier",
                   "tokens": n, "layers": L, "budget": cfg.budget, "paged_block": bs},
        "pack_unpack_pct_hbm": round((pack_bytes + unpack_bytes) / (t_pack + t_unpack) / 1e9
                                     / HBM_PEAK_GBS, 4),
        "score_tflops": round(score_tflops, 1),
        "score_pct_mfma": round(score_tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "stage_ms_per_step": {s: round(v, 4) for s, v in per_step_ms.items()},
        "stage_ms_median": {s: round(float(np.median(v)), 4) for s, v in step_ms.items()},
        "stage_ms_min": {s: round(float(v.min()), 4) for s, v in step_ms.items()},
        "cold_cache": "1 GiB write before pack, unpack and paged unpack",
        "payload_bytes": plan.payload_bytes,
        "counts": {"fp16": plan.n16, "int8": plan.n8, "int4": plan.n4},
        "roofline": {"bound": "mfma", "kernel": kernel_name, "achieved": round(ach, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": counted_traffic(kernel_name, cfg.name),
                     "flops_per_launch": pass_flops,
                     "avg_launch_ms": round(mean_launch[dom], 4)},
        "roofline_stages": {"pack": rl(pack_bytes, t_pack, f"pack_kernel<{d},{nb}>"),
                            "unpack": rl(unpack_bytes, t_unpack, f"unpack_kernel<{d},{nb},false>"),
                            "unpack_paged": rl(unpack_bytes, t_paged,
                                               f"unpack_kernel<{d},{nb},true>")},
        "variants": {"kvnorm": rl(kv_bytes // 2 + 4 * n, t_kvnorm, f"kvnorm_kernel<{d}>"),
                     # n = 8192 elements: one launch's latency, not a bandwidth figure
                     "recency": {"bound": "latency", "kernel": "recency_kernel",
                                 "us_per_launch": round(t_recency * 1e6, 2)}},
        "upgrade": {"tokens": n_up,
                    "pack": rl(up_bytes, t_up_pack, f"upgrade_pack_kernel<{d},{nb}>"),
                    "unpack_paged": rl(up_bytes, t_up_paged,
                                       f"upgrade_unpack_kernel<{d},{nb},true>")},
        # whole sk_decode_attention calls (one partial launch per sent tier,
        # then the merge): bytes and time of the call, not of one kernel
        "decode": {"layers": L,
                   "payload": call_rl(dec_bytes, t_dec),
                   "fp16_payload": call_rl(dec16_bytes, t_dec16),
                   "ms": round(t_dec * 1e3, 4), "fp16_ms": round(t_dec16 * 1e3, 4),
                   "speedup_vs_fp16": round(t_dec16 / t_dec, 3)},
        "score_other_shapes": score_shapes,
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "copy_bytes": int(src.numel()),
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def score_kernel_names(Hq, Hkv, d):
    """Template instances the library launches for this shape (the rule of
    its launchers: W = the largest of 4, 2, 1 dividing Hq/Hkv heads per
    row-pass workgroup, QW = 4/W blocks of 64 queries, stages of 64 rows,
    32 at d = 256; the column pass uses 4 wavefronts)."""
    R = Hq // Hkv
    W = next(w for w in (4, 2, 1) if R % w == 0)
    QW = 4 // W
    KS = 32 if d == 256 else 64
    return {"rowlse": f"rowlse_kernel<{d},{W},{QW},{KS}>",
            "colsum": f"colsum_kernel<{d},4,{KS}>"}


def pack_batch(Hkv, d):
    """Rows steps whose loads the pack/unpack kernels batch per token (the
    power of two, up to 8, covering 2*Hkv rows at 64/(d/8) rows a step)."""
    rpp = 64 // (d // 8)
    steps = (2 * Hkv + rpp - 1) // rpp
    nb = 1
    while nb < steps and nb < 8:
        nb *= 2
    return nb


def counted_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summaries (FETCH_SIZE + WRITE_SIZE, calibrated against a
    device copy), or None when no summary covers it or its source file changed
    since."""
    import glob
    import hashlib
    import re

    root = os.path.dirname(os.path.abspath(__file__))
    pat = re.compile(r"<!-- traffic workload=(\S+) kernel=(\S+) bytes_per_launch=(\d+) "
                     r"source=(\S+) sha256=([0-9a-f]+) -->")
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*.md"))):
        for m in pat.finditer(open(path).read()):
            if m.group(1) != workload or m.group(2) != kernel:
                continue
            src = os.path.join(root, m.group(4))
            if not os.path.exists(src):
                continue
            if hashlib.sha256(open(src, "rb").read()).hexdigest() == m.group(5):
                return int(m.group(3))
    return None


def cpu_baseline(cfg, budget_s):
    """The oracle, as it stands, timed on the host cores on a bounded sample of
    the same workload; reported in the metric's unit."""
    from oracle import assign as OA, plan as OP, quant as OQ, score as OS
    from workloads import gen

    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    L, Hq, Hkv, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    opl = OP.make_plan(L, Hq, Hkv, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    # pack + unpack of whole layers until about half the budget is spent
    k = gen.keys(cfg, 0)
    v = gen.values(cfg, 0)
    s32 = np.random.default_rng(0).random(n).astype(np.float32)
    t0 = time.time()
    _, _, amap, _ = OA.assign(s32, opl.n16, opl.n8, opl.n4, opl.sinks)
    t_assign = time.time() - t0
    layers = 0
    t_pu = 0.0
    buf = np.zeros(opl.payload_bytes, dtype=np.uint8)
    while t_pu < budget_s / 2 and layers < L:
        t0 = time.time()
        for off, data in OQ.pack_layer(k, v, layers, amap, opl):
            buf[off:off + data.size] = data
        OQ.unpack_layer(buf, layers, amap, opl, Hkv, d)
        t_pu += time.time() - t0
        layers += 1
    kv_layer = 2 * n * Hkv * d * 2
    gbs = 2 * kv_layer * layers / t_pu / 1e9
    # score: whole (layer, head) pairs in fp64 until the other half is spent
    q = gen.queries(cfg, 0, k=k)
    heads = 0
    t_sc = 0.0
    while t_sc < budget_s / 2 and heads < Hq:
        t0 = time.time()
        OS.head_column_sums(q[:, heads, :], k[:, heads // (Hq // Hkv), :])
        t_sc += time.time() - t0
        heads += 1
    tflops = heads * d * n * (n + 1) / t_sc / 1e12          # single-pass QK^T count
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"pack+unpack of {layers} of {L} layers (fp16-equiv GB/s, numpy, "
                      f"1 thread); score of {heads} (layer, head) pairs of {L * Hq} in fp64",
            "score_tflops": round(tflops, 6), "assign_s_full": round(t_assign, 3)}


if __name__ == "__main__":
    main()
