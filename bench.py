"""Benchmark of the mixed-precision KV transfer path on one MI355X.

One step = the whole path over the batched serving mix, the largest workload
that fits one GPU: 16 Mistral-7B-shaped requests (32 layers, 32 query / 8 KV
heads, head dim 128) with seeded log-uniform lengths in [1024, 65536]
(277,716 tokens), S = 4 sinks, 3-tier.  Per request and layer the two score
passes (row log-sum-exp, then the MFMA column sums accumulated into the
request's score); then, at each budget of the sweep b in {0.3, 0.5, 0.7}, the
tier assignment of every request, the pack of every request, and the paged
unpack of every request into one shared fp16 cache of 16-token blocks under a
seeded permuted block table.  Inputs are seeded synthetic tensors drawn on
the device (workloads.gen_device), resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the fp16-equivalent KV throughput of pack
+ unpack over the step, sum(2 * KV_fp16_bytes) / sum(t_pack + t_unpack) over
every request and budget, from HIP events recorded on the launch stream
around every launch inside the timed steps; the score's TFLOP/s and every
stage's time are reported beside it.  The single-request workloads
(Gemma-2-9B-, Qwen2.5-7B- and Mistral-7B-shaped) follow under ``workloads``,
each as its own whole-path measurement with its own rooflines.
"""

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "KV pack+unpack GB/s (fp16-equiv, % HBM peak); importance-score TFLOP/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="batched_mix",
                    help="the headline workload (batched_mix, or a single-request one)")
    ap.add_argument("--others", default="gemma2_9b,qwen25_7b_2tier,mistral7b",
                    help="comma-separated single-request workloads measured after the "
                         "headline ('' for none)")
    ap.add_argument("--other-steps", type=int, default=3,
                    help="timed steps of each single-request workload at least; more when "
                         "that many take under 1 s (up to 20)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="rough budget of the oracle's timed sample")
    ap.add_argument("--score-launch", choices=("layers", "per-layer"), default="layers",
                    help="score passes as one launch over all layers of a request, or one "
                         "launch per layer (the same results, bit for bit)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Marks:
    """HIP events around every launch of a step, on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.rec = []

    def __call__(self, stage, work, fn):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.rec.append((stage, work, a, b))

    def collect(self):
        out = {}
        for stage, work, a, b in self.rec:
            ms, w = out.setdefault(stage, ([], []))
            ms.append(a.elapsed_time(b))
            w.append(work)
        return {s: (np.array(ms), np.array(w, dtype=np.float64)) for s, (ms, w) in out.items()}


def untimed(stage, work, fn):
    fn()


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
    """Row steps whose loads the pack/unpack kernels batch per token (the
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


def step_spread(res, stages):
    """Median and minimum over the timed steps of each stage's per-step time
    (ms): res holds one {launch label: (ms array, work array)} per step and
    a stage sums the launches of its labels within a step."""
    out = {}
    for name, labels in stages.items():
        per_step = np.array([sum(float(r_[k][0].sum()) for k in labels) for r_ in res])
        out[name] = [round(float(np.median(per_step)), 4), round(float(per_step.min()), 4)]
    return out


def hbm_rl(bytes_, sec, kernel, workload, launches=1):
    """Roofline entry of an HBM-bound kernel: algorithmic bytes per launch
    over its average launch time."""
    gbs = bytes_ / sec / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": int(round(bytes_ / launches)),
            "avg_launch_ms": round(sec * 1e3 / launches, 4),
            "traffic": counted_traffic(kernel, workload)}


def mfma_rl(flops, ms, kernel, workload):
    """Roofline entry of a score pass: causal single-pass QK^T flops per
    launch (2 d per causal pair and query head) over its average launch
    time, both averaged over the launches of the timed steps."""
    ach = flops.sum() / (ms.sum() * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(ach, 1),
            "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": counted_traffic(kernel, workload),
            "flops_per_launch": float(flops.mean()), "avg_launch_ms": round(float(ms.mean()), 4),
            "launches_per_step": None}


def torch_copy_gbs(torch, nbytes, dev):
    """torch's device-to-device copy of `nbytes` (r + w bytes / time): a
    reference point, and the calibration kernel of the counter runs."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * 3 / (c0.elapsed_time(c1) * 1e-3) / 1e9


def score_passes(m, sk, per_layer, shape, Q, K, lse, score, cws, pass_flops):
    """Both score passes of one request, every layer: one launch per pass
    (sk_score_rowlse_layers / sk_score_colsum_layers) or, with per_layer, a
    launch per layer and pass.  lse is [L][Hq][n] (rows of layer 0 are used
    by the per-layer form); each mark carries the flops of what it launched."""
    L = shape.n_layers
    if not per_layer:
        m("rowlse", L * pass_flops, lambda: sk.score_rowlse_layers(shape, Q, K, lse))
        m("colsum", L * pass_flops,
          lambda: sk.score_colsum_layers(shape, Q, K, lse, score, False, cws))
        return
    shape1 = sk.Shape(1, shape.n_q_heads, shape.n_kv_heads, shape.head_dim)
    for layer in range(L):
        m("rowlse", pass_flops, lambda: sk.score_rowlse(shape1, Q[layer], K[layer], lse[0]))
        m("colsum", pass_flops, lambda: sk.score_colsum(shape1, Q[layer], K[layer], lse[0],
                                                        score, layer > 0, cws))


def score_buffers(torch, sk, shape, n, per_layer, dev):
    """lse [L][Hq][n] and the colsum workspace for a request of n tokens."""
    shape1 = sk.Shape(1, shape.n_q_heads, shape.n_kv_heads, shape.head_dim)
    L = 1 if per_layer else shape.n_layers
    ws = (sk.colsum_workspace_bytes(shape1, n) if per_layer
          else sk.colsum_layers_workspace_bytes(shape, n))
    return (torch.empty(L * shape.n_q_heads * n, dtype=torch.float32, device=dev),
            torch.empty(max(1, ws), dtype=torch.uint8, device=dev))


# --------------------------------------------------------------- batched mix --

def run_batched(cfg, args, dev, torch, sk):
    from workloads import gen, gen_device as gd

    L, Hq, Hkv, d, bs = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
    lengths = gen.request_lengths(cfg)
    tables, num_blocks = gen.block_tables(cfg, lengths)
    R = len(lengths)
    nmax = max(lengths)
    shape = sk.Shape(L, Hq, Hkv, d)
    per_layer = args.score_launch == "per-layer"
    pols = {b: [sk.Policy(n, cfg.sinks, cfg.three_tier, b) for n in lengths] for b in cfg.budgets}
    plans = {b: [sk.plan_make(shape, p) for p in pols[b]] for b in cfg.budgets}
    kv = [2 * L * n * Hkv * d * 2 for n in lengths]
    need = (sum(n * L * (Hq + 4 * Hkv) * d * 2 for n in lengths)
            + sum(max(plans[b][r].payload_bytes for b in cfg.budgets) for r in range(R))
            + (1 << 30))
    free, total = torch.cuda.mem_get_info(dev)
    log(f"batched mix: {R} requests, {sum(lengths)} tokens, lengths {lengths}; "
        f"{need / 1e9:.1f} GB of device memory ({free / 1e9:.1f} GB free)")
    if need > free:
        raise SystemExit(f"the batched mix needs {need / 1e9:.1f} GB, {free / 1e9:.1f} GB free")

    t0 = time.time()
    Q, K, V = [], [], []
    for r, n in enumerate(lengths):
        Q.append(torch.empty((L, n, Hq, d), dtype=torch.float16, device=dev))
        K.append(torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev))
        V.append(torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev))
        for layer in range(L):
            gd.keys(cfg, layer, n, r, out=K[r][layer])
            gd.values(cfg, layer, n, r, out=V[r][layer])
            gd.queries(cfg, layer, n, r, k=K[r][layer], out=Q[r][layer])
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f} s")

    lse_all, cws = score_buffers(torch, sk, shape, nmax, per_layer, dev)
    lse = [lse_all[:lse_all.numel() // nmax * n].view(-1, Hq, n) for n in lengths]
    score = [torch.empty(n, dtype=torch.float32, device=dev) for n in lengths]
    amap = [torch.empty(n, dtype=torch.int32, device=dev) for n in lengths]
    order = [torch.empty(n, dtype=torch.int32, device=dev) for n in lengths]
    payload = [torch.empty(max(plans[b][r].payload_bytes for b in cfg.budgets),
                           dtype=torch.uint8, device=dev) for r in range(R)]
    btab = [torch.from_numpy(t).to(dev) for t in tables]
    Kc = torch.empty((L, num_blocks, bs, Hkv, d), dtype=torch.float16, device=dev)
    Vc = torch.empty_like(Kc)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    pass_flops = [Hq * d * n * (n + 1) for n in lengths]         # one pass, one layer

    def pbytes(b, r):
        n = lengths[r]
        return kv[r] + 4 * n + plans[b][r].payload_bytes                     # K,V + map -> P

    def ubytes(b, r):
        n = lengths[r]
        return plans[b][r].payload_bytes + 4 * n + 4 * len(tables[r]) + kv[r]  # P + map + bt -> KV

    def step(m):
        for r in range(R):
            score_passes(m, sk, per_layer, shape, Q[r], K[r], lse[r], score[r], cws,
                         pass_flops[r])
        for b in cfg.budgets:
            for r in range(R):
                m(f"assign@{b}", 0,
                  lambda: sk.assign_tiers(pols[b][r], plans[b][r], score[r], amap[r], order[r]))
            scratch.fill_(0x5A)      # evict the Infinity Cache before the pack phase
            for r in range(R):
                m(f"pack@{b}", pbytes(b, r),
                  lambda: sk.pack(shape, plans[b][r], K[r], V[r], amap[r], order[r],
                                  payload[r][:plans[b][r].payload_bytes]))
            scratch.fill_(0x5A)
            for r in range(R):
                m(f"unpack_paged@{b}", ubytes(b, r),
                  lambda: sk.unpack_paged(shape, plans[b][r],
                                          payload[r][:plans[b][r].payload_bytes], amap[r],
                                          Kc, Vc, btab[r], bs))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(untimed)
    torch.cuda.synchronize()
    marks = [Marks(torch) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    wall0 = time.time()
    start.record()
    for i in range(args.steps):
        step(marks[i])
        log(f"step {i + 1} enqueued")
    end.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps
    res = [m.collect() for m in marks]

    def cat(stage):
        return (np.concatenate([r_[stage][0] for r_ in res]),
                np.concatenate([r_[stage][1] for r_ in res]))

    K_ = args.steps
    t_pack = sum(cat(f"pack@{b}")[0].sum() for b in cfg.budgets) * 1e-3 / K_
    t_unp = sum(cat(f"unpack_paged@{b}")[0].sum() for b in cfg.budgets) * 1e-3 / K_
    kv_total = sum(kv)
    nb_ = len(cfg.budgets)
    value = 2 * kv_total * nb_ / (t_pack + t_unp) / 1e9
    moved = sum(pbytes(b, r) + ubytes(b, r) for b in cfg.budgets for r in range(R))
    rms, rfl = cat("rowlse")
    cms, cfl = cat("colsum")
    score_s = (rms.sum() + cms.sum()) * 1e-3 / K_
    score_flops = 2 * L * sum(pass_flops)
    score_tflops = score_flops / score_s / 1e12
    names = score_kernel_names(Hq, Hkv, d)
    dom = "colsum" if cms.sum() >= rms.sum() else "rowlse"
    roof = mfma_rl(*((cfl, cms) if dom == "colsum" else (rfl, rms)), names[dom], cfg.name)
    roof["launches_per_step"] = R * (L if per_layer else 1)
    nbk = pack_batch(Hkv, d)

    per_budget = {}
    for b in cfg.budgets:
        pm, _ = cat(f"pack@{b}")
        um, _ = cat(f"unpack_paged@{b}")
        am, _ = cat(f"assign@{b}")
        tp, tu = pm.sum() * 1e-3 / K_, um.sum() * 1e-3 / K_
        pb = sum(pbytes(b, r) for r in range(R))
        ub = sum(ubytes(b, r) for r in range(R))
        # per request, over all steps: launch r of each step
        pms = pm.reshape(K_, R).mean(axis=0)
        ums = um.reshape(K_, R).mean(axis=0)
        per_req_b = [{"n": lengths[r], "pack_ms": round(float(pms[r]), 4),
                      "pack_frac": round(pbytes(b, r) / (pms[r] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "unpack_paged_ms": round(float(ums[r]), 4),
                      "unpack_paged_frac": round(ubytes(b, r) / (ums[r] * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 4)} for r in range(R)]
        per_budget[str(b)] = {
            "per_request": per_req_b,
            "payload_bytes": sum(plans[b][r].payload_bytes for r in range(R)),
            "counts": [int(sum(getattr(plans[b][r], f) for r in range(R)))
                       for f in ("n16", "n8", "n4")],
            "fp16_equiv_gbs": round(2 * kv_total / (tp + tu) / 1e9, 1),
            "pack": hbm_rl(pb, tp, f"pack_kernel<{d},{nbk}>", f"{cfg.name}@{b}", R),
            "unpack_paged": hbm_rl(ub, tu, f"unpack_kernel<{d},{nbk},true>", f"{cfg.name}@{b}", R),
            "assign_ms_per_step": round(am.sum() / K_, 4)}

    # score efficiency per request (its launches over all steps)
    per_req = []
    nrl = len(rms) // K_ // R            # launches per pass and request: 1, or L
    for r, n in enumerate(lengths):
        idx = np.concatenate([np.arange(s * R * nrl + r * nrl, s * R * nrl + (r + 1) * nrl)
                              for s in range(K_)])
        f = L * pass_flops[r] * K_
        per_req.append({"n": n, "rowlse_ms": round(float(rms[idx].mean()), 4),
                        "colsum_ms": round(float(cms[idx].mean()), 4),
                        "rowlse_frac": round(f / (rms[idx].sum() * 1e-3) / 1e12
                                             / MFMA_F16_PEAK_TFLOPS, 4),
                        "colsum_frac": round(f / (cms[idx].sum() * 1e-3) / 1e12
                                             / MFMA_F16_PEAK_TFLOPS, 4)})

    line = {
        "metric": METRIC,
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
        "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": f"{cfg.name}: {R} requests of Mistral-7B shape (L={L} Hq={Hq} "
                               f"Hkv={Hkv} d={d}), lengths log-uniform in [{cfg.len_lo}, "
                               f"{cfg.len_hi}] ({sum(lengths)} tokens), S={cfg.sinks}, 3-tier, "
                               f"b in {list(cfg.budgets)}, paged unpack ({bs}-token blocks)",
                   "requests": R, "tokens": sum(lengths), "lengths": lengths, "layers": L,
                   "budgets": list(cfg.budgets), "paged_block": bs,
                   "kv_fp16_bytes": kv_total},
        "pack_unpack_pct_hbm": round(moved / (t_pack + t_unp) / 1e9 / HBM_PEAK_GBS, 4),
        "score_tflops": round(score_tflops, 1),
        "score_pct_mfma": round(score_tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "score_flops_per_step": float(score_flops),
        # the single-pass q.k count (half the two passes' flops), and the
        # exponentials: one per causal (query, key) pair and pass
        "score_tflops_single_pass": round(score_tflops / 2, 1),
        "score_exps_per_step": float(score_flops / (2 * d)),
        "score_gexp_per_s": round(score_flops / (2 * d) / score_s / 1e9, 1),
        "roofline": roof,
        "roofline_other_pass": dict(mfma_rl(*((rfl, rms) if dom == "colsum" else (cfl, cms)),
                                            names["rowlse" if dom == "colsum" else "colsum"],
                                            cfg.name),
                                    launches_per_step=roof["launches_per_step"]),
        "score_launch": "one launch per pass and layer" if per_layer else
                        "one launch per pass over all layers of a request",
        "stage_ms_per_step": {"rowlse": round(rms.sum() / K_, 3),
                              "colsum": round(cms.sum() / K_, 3),
                              "pack": round(t_pack * 1e3, 3),
                              "unpack_paged": round(t_unp * 1e3, 3)},
        "stage_ms_median_min": step_spread(res, {
            "rowlse": ["rowlse"], "colsum": ["colsum"],
            "pack": [f"pack@{b}" for b in cfg.budgets],
            "unpack_paged": [f"unpack_paged@{b}" for b in cfg.budgets]}),
        "budgets": per_budget,
        "score_per_request": per_req,
        "cold_cache": "1 GiB write before each pack phase and each unpack phase",
        "wall_s_timed": round(wall, 3),
    }
    del Q, K, V, Kc, Vc, payload, scratch, lse_all, cws
    return line, lengths


# ----------------------------------------------------------- single request --

def run_single(cfg, steps, warmup, dev, torch, sk, extras, per_layer=False, adapt=False):
    from workloads import gen_device as gd

    L, Hq, Hkv, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    log(f"workload {cfg.name}: L={L} Hq={Hq} Hkv={Hkv} d={d} n={n}")
    t0 = time.time()
    Q = torch.empty((L, n, Hq, d), dtype=torch.float16, device=dev)
    K = torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev)
    V = torch.empty((L, n, Hkv, d), dtype=torch.float16, device=dev)
    for layer in range(L):
        gd.keys(cfg, layer, n, out=K[layer])
        gd.values(cfg, layer, n, out=V[layer])
        gd.queries(cfg, layer, n, k=K[layer], out=Q[layer])
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f} s")

    shape = sk.Shape(L, Hq, Hkv, d)
    pol = sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget)
    plan = sk.plan_make(shape, pol)
    lse, cws = score_buffers(torch, sk, shape, n, per_layer, dev)
    lse = lse.view(-1, Hq, n)
    score = torch.empty(n, dtype=torch.float32, device=dev)
    amap = torch.empty(n, dtype=torch.int32, device=dev)
    order = torch.empty(n, dtype=torch.int32, device=dev)
    payload = torch.empty(plan.payload_bytes, dtype=torch.uint8, device=dev)
    Ko = torch.empty_like(K)
    Vo = torch.empty_like(V)
    bs = 16
    nblk = (n + bs - 1) // bs
    block_table = torch.from_numpy(
        np.random.default_rng(0).permutation(nblk).astype(np.int32)).to(dev)
    Kc = torch.empty((L, nblk, bs, Hkv, d), dtype=torch.float16, device=dev)
    Vc = torch.empty_like(Kc)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    kv_bytes = 2 * L * n * Hkv * d * 2
    pass_flops = Hq * d * n * (n + 1)
    pack_bytes = kv_bytes + 4 * n + plan.payload_bytes
    unpack_bytes = plan.payload_bytes + 4 * n + kv_bytes
    paged_bytes = unpack_bytes + 4 * nblk

    def step(m):
        score_passes(m, sk, per_layer, shape, Q, K, lse, score, cws, pass_flops)
        m("assign", 0, lambda: sk.assign_tiers(pol, plan, score, amap, order))
        scratch.fill_(0x5A)
        m("pack", pack_bytes, lambda: sk.pack(shape, plan, K, V, amap, order, payload))
        scratch.fill_(0x5A)
        m("unpack", unpack_bytes, lambda: sk.unpack(shape, plan, payload, amap, Ko, Vo))
        scratch.fill_(0x5A)
        m("unpack_paged", paged_bytes,
          lambda: sk.unpack_paged(shape, plan, payload, amap, Kc, Vc, block_table, bs))

    for _ in range(warmup):
        step(untimed)
    if adapt:
        # a nested workload: one more untimed step, timed whole, sets the
        # step count, at least `steps` and enough for 1 s of timed work, up
        # to 20 steps (a headline run times exactly the steps asked for)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        step(untimed)
        c1.record()
        torch.cuda.synchronize()
        steps = max(steps, min(20, int(np.ceil(1000.0 / max(c0.elapsed_time(c1), 1e-3)))))
    torch.cuda.synchronize()
    marks = [Marks(torch) for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(marks[i])
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    res = [m.collect() for m in marks]

    def cat(stage):
        return (np.concatenate([r_[stage][0] for r_ in res]),
                np.concatenate([r_[stage][1] for r_ in res]))

    per = {s: cat(s)[0].sum() * 1e-3 / steps for s in
           ("rowlse", "colsum", "assign", "pack", "unpack", "unpack_paged")}
    rms, rfl = cat("rowlse")
    cms, cfl = cat("colsum")
    names = score_kernel_names(Hq, Hkv, d)
    dom = "colsum" if cms.sum() >= rms.sum() else "rowlse"
    score_tflops = 2 * L * pass_flops / (per["rowlse"] + per["colsum"]) / 1e12
    nbk = pack_batch(Hkv, d)
    out = {
        "config": {"workload": f"{cfg.name}: L={L} Hq={Hq} Hkv={Hkv} d={d} n={n} S={cfg.sinks} "
                               f"b={cfg.budget} {'3' if cfg.three_tier else '2'}-tier",
                   "tokens": n, "layers": L, "budget": cfg.budget, "paged_block": bs},
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 3),
        "value": round(2 * kv_bytes / (per["pack"] + per["unpack"]) / 1e9, 1),
        "unit": "GB/s (fp16-equiv pack + dense unpack)",
        "pack_unpack_pct_hbm": round((pack_bytes + unpack_bytes) / (per["pack"] + per["unpack"])
                                     / 1e9 / HBM_PEAK_GBS, 4),
        "score_tflops": round(score_tflops, 1),
        "score_pct_mfma": round(score_tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "score_tflops_single_pass": round(score_tflops / 2, 1),
        "score_exps_per_step": float(L * pass_flops / d),
        "score_gexp_per_s": round(L * pass_flops / d / (per["rowlse"] + per["colsum"]) / 1e9, 1),
        "roofline": dict(mfma_rl(*((cfl, cms) if dom == "colsum" else (rfl, rms)), names[dom],
                                 cfg.name), launches_per_step=L if per_layer else 1),
        "roofline_other_pass": dict(mfma_rl(*((rfl, rms) if dom == "colsum" else (cfl, cms)),
                                            names["rowlse" if dom == "colsum" else "colsum"],
                                            cfg.name), launches_per_step=L if per_layer else 1),
        "roofline_stages": {
            "pack": hbm_rl(pack_bytes, per["pack"], f"pack_kernel<{d},{nbk}>", cfg.name),
            "unpack": hbm_rl(unpack_bytes, per["unpack"], f"unpack_kernel<{d},{nbk},false>",
                             cfg.name),
            "unpack_paged": hbm_rl(paged_bytes, per["unpack_paged"],
                                   f"unpack_kernel<{d},{nbk},true>", cfg.name)},
        "stage_ms_per_step": {s: round(v * 1e3, 4) for s, v in per.items()},
        "stage_ms_median_min": step_spread(res, {s: [s] for s in per}),
        "payload_bytes": plan.payload_bytes,
        "counts": {"fp16": plan.n16, "int8": plan.n8, "int4": plan.n4},
        "cold_cache": "1 GiB write before pack, unpack and paged unpack",
    }

    def timed(fn, reps):
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3

    reps = 5
    # decode attention straight from the payload, all layers in one call (one
    # decode query per layer): whole calls, one partial launch per sent tier
    # plus the merge; the per-kernel times are in the rocprofv3 summaries
    qdec = torch.from_numpy((np.random.default_rng(2).standard_normal((L, Hq, d)) * 0.5)
                            .astype(np.float16)).to(dev)
    odec = torch.empty((L, Hq, d), dtype=torch.float32, device=dev)
    ldec = torch.empty((L, Hq), dtype=torch.float32, device=dev)
    dws = torch.empty(max(1, sk.decode_workspace_bytes(shape, plan, L)), dtype=torch.uint8,
                      device=dev)
    t_dec = timed(lambda: sk.decode_attention(shape, plan, payload, qdec, odec, ldec, ws=dws),
                  reps)
    dec_bytes = plan.payload_bytes + L * Hq * d * (2 + 4) + L * Hq * 4
    out["decode"] = {"layers": L, "call": "sk_decode_attention",
                     "achieved": round(dec_bytes / t_dec / 1e9, 1), "unit": "GB/s",
                     "frac": round(dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes_per_call": dec_bytes, "ms": round(t_dec * 1e3, 4)}
    if extras:
        alt = torch.empty(n, dtype=torch.float32, device=dev)
        t_kvnorm = timed(lambda: sk.score_kvnorm(shape, K, alt), reps)
        t_recency = timed(lambda: sk.recency_weight(score, 1e-3, alt), reps)
        n_up = n // 8
        up_tokens = torch.from_numpy(
            np.random.default_rng(1).choice(n, size=n_up, replace=False).astype(np.int32)).to(dev)
        up_payload = torch.empty(sk.upgrade_bytes(shape, n_up), dtype=torch.uint8, device=dev)
        t_up_pack = timed(lambda: sk.upgrade_pack(shape, K, V, up_tokens, up_payload), reps)
        t_up_paged = timed(lambda: sk.upgrade_unpack_paged(shape, n, up_payload, up_tokens, Kc,
                                                           Vc, block_table, bs), reps)
        up_bytes = 2 * up_payload.numel() + 4 * n_up
        out["variants"] = {"kvnorm": hbm_rl(kv_bytes // 2 + 4 * n, t_kvnorm,
                                            f"kvnorm_kernel<{d}>", cfg.name),
                           "recency": {"bound": "latency", "kernel": "recency_kernel",
                                       "us_per_launch": round(t_recency * 1e6, 2)}}
        out["upgrade"] = {"tokens": n_up,
                          "pack": hbm_rl(up_bytes, t_up_pack, f"upgrade_pack_kernel<{d},{nbk}>",
                                         cfg.name),
                          "unpack_paged": hbm_rl(up_bytes, t_up_paged,
                                                 f"upgrade_unpack_kernel<{d},{nbk},true>",
                                                 cfg.name)}
        out["torch_copy_gbs"] = round(torch_copy_gbs(torch, 512 << 20, dev), 1)
    del Q, K, V, Ko, Vo, Kc, Vc, payload, scratch
    return out


# ------------------------------------------------------------- CPU baseline --

def cpu_baseline(cfg, lengths, budget_s):
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
    L, Hq, Hkv, d = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim
    if lengths:
        r = int(np.argmin([abs(n - 8192) for n in lengths]))   # a mid-length request
        n, b = lengths[r], 0.5
    else:
        r, n, b = 0, cfg.tokens, cfg.budget
    opl = OP.make_plan(L, Hq, Hkv, d, n, cfg.sinks, b, cfg.three_tier)
    k = gen.keys(cfg, 0, n, request=r)
    v = gen.values(cfg, 0, n, request=r)
    s32 = np.random.default_rng(0).random(n).astype(np.float32)
    t0 = time.time()
    _, _, amap, _ = OA.assign(s32, opl.n16, opl.n8, opl.n4, opl.sinks)
    t_assign = time.time() - t0
    layers, t_pu = 0, 0.0
    buf = np.zeros(opl.payload_bytes, dtype=np.uint8)
    bs = cfg.block_size
    nblk = (n + bs - 1) // bs
    bt = np.arange(nblk, dtype=np.int32)
    kc = np.zeros((1, nblk, bs, Hkv, d), dtype=np.float16)
    vc = np.zeros_like(kc)
    while t_pu < budget_s / 2 and layers < L:
        t0 = time.time()
        for off, data in OQ.pack_layer(k, v, layers, amap, opl):
            buf[off:off + data.size] = data
        kk, vv = OQ.unpack_layer(buf, layers, amap, opl, Hkv, d)
        j = np.arange(n)
        kc[0, bt[j // bs], j % bs] = kk
        vc[0, bt[j // bs], j % bs] = vv
        t_pu += time.time() - t0
        layers += 1
    kv_layer = 2 * n * Hkv * d * 2
    gbs = 2 * kv_layer * layers / t_pu / 1e9
    q = gen.queries(cfg, 0, n, request=r, k=k)
    heads, t_sc = 0, 0.0
    while t_sc < budget_s / 2 and heads < Hq:
        t0 = time.time()
        OS.head_column_sums(q[:, heads, :], k[:, heads // (Hq // Hkv), :])
        t_sc += time.time() - t0
        heads += 1
    tflops = heads * d * n * (n + 1) / t_sc / 1e12          # single-pass QK^T count
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"request {r} (n={n}) of {cfg.name}: pack+unpack of {layers} of {L} "
                      f"layers at b={b} (fp16-equiv GB/s, numpy, 1 thread); score of {heads} "
                      f"(layer, head) pairs of {L * Hq} in fp64 (BLAS threads)",
            "score_tflops": round(tflops, 6), "assign_s_one_request": round(t_assign, 3)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the transfer path is built and timed on a "
              "single MI355X (multi-GPU sharding is a design note, not a measured path).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import serving_sk_score_amd as sk
    from workloads import get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sk.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda", 0)
    cfg = get_config(args.workload)
    if cfg.requests:
        line, lengths = run_batched(cfg, args, dev, torch, sk)
    else:
        one = run_single(cfg, args.steps, args.warmup, dev, torch, sk, extras=True,
                         per_layer=args.score_launch == "per-layer")
        lengths = None
        line = {"metric": METRIC, "value": one.pop("value"), "unit": "GB/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": one.pop("ms_per_step"),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "f16", "data": "synthetic (seeded, drawn on the device)", **one}
    gc.collect()
    torch.cuda.empty_cache()
    others = [w for w in args.others.split(",") if w and w != cfg.name]
    if others:
        line["workloads"] = {}
        for w in others:
            line["workloads"][w] = run_single(get_config(w), args.other_steps, 1, dev, torch, sk,
                                              extras=(w == "mistral7b"),
                                              per_layer=args.score_launch == "per-layer",
                                              adapt=True)
            gc.collect()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, lengths, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
