"""Benchmark of one Sparse VideoGen attention layer on one MI355X.

A step is one pass of the whole path over the resident inputs of one layer:
online profiling on 1 % sampled rows -> key-tile lists -> token-major layout
transformation of the temporal heads' Q, K, V -> block-banded sparse
attention -> inverse transformation of their output.  Default workload: the
HunyuanVideo-shaped layer (33 frames x 3600 tokens = 118,800 tokens, 24 heads,
d = 128, bf16, a1 = 2, a2 = 160).

Prints one JSON line.  ``value`` is the effective throughput of the whole
step, 4*d*(active query-key pairs) / step time, in TFLOP/s; ``attn_*`` fields
give the sparse-attention kernel alone (the a5 figure), measured with HIP
events on the stream the kernels run on.

  python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu]
                  [--virtual] [--calib-copy] [--search]

--search also times the Sparse-vDiT offline mode search (svg_search_modes:
full, window, temporal-band and stripe attention of the sampled rows, 1 % of
the video rows when the workload samples none) on the same inputs and adds
search_* fields.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# fp8 scores + bf16 P.V: half the attention FLOPs at each rate
PEAK_FP8_QK_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def pair_count(N, F, T, mode, a1=1, a2=1, window=1, stripe=1):
    """Active (query, key) pairs of one head, from the masks' closed forms.

    Video-video pairs: spatial F^2 (N + 2 sum_{k=1}^{a1-1} (N-k)), temporal
    N^2 (F + 2 sum_{k=1}^{a2-1} (F-k)) (thresholds clipped to N, F), window
    n(2W-1) - W(W-1) for W < n = N*F, stripe n*min(S, n), full n^2; plus the
    dense text rows and columns T*L + n*T; skip heads have none."""
    SPATIAL, TEMPORAL, FULL, SKIP, WINDOW, STRIPE = range(6)
    n = N * F
    L = T + n
    if mode == SKIP:
        return 0
    text = T * L + n * T
    if mode == SPATIAL:
        a = min(a1, N)
        vid = F * F * (N + 2 * sum(N - k for k in range(1, a)))
    elif mode == TEMPORAL:
        a = min(a2, F)
        vid = N * N * (F + 2 * sum(F - k for k in range(1, a)))
    elif mode == FULL:
        vid = n * n
    elif mode == WINDOW:
        W = min(window, n)
        vid = n * (2 * W - 1) - W * (W - 1)
    elif mode == STRIPE:
        vid = n * min(stripe, n)
    else:
        raise ValueError(mode)
    return text + vid


CSRC = os.path.join(ROOT, "sparse_attention_video_svg_amd", "csrc")
# the sources each timed kernel is built from: a committed counter record is
# used only while the hash of its kernel's sources is the one it was taken at
KERNEL_SOURCES = {
    "k_attn_bf16": ("attn_bf16.hip", "attn_common.h", "svg_device.h", "svg_internal.h", "svg_sched.h"),
    "k_attn_fp8": ("attn_fp8.hip", "attn_common.h", "svg_device.h", "svg_internal.h", "svg_sched.h"),
    "k_svg2_attn": ("svg2.hip", "attn_common.h", "svg_device.h", "svg_internal.h", "svg_sched.h"),
    "k_permute": ("permute.hip", "svg_device.h", "svg_internal.h"),
    "k_prof_sweep": ("attn_bf16.hip", "attn_common.h", "profile.hip", "svg_device.h", "svg_internal.h",
                     "svg_sched.h"),
}
# rocprofv3 summaries under profiles/ holding an HBM-traffic record, by
# (timed kernel, workload, layout)
TRAFFIC_RECORDS = {
    ("k_attn_bf16", 1, "explicit"): "k_attn_bf16_cogvideox_13x4080_h48_d64.md",
    ("k_attn_bf16", 2, "explicit"): "k_attn_bf16_hunyuanvideo_33x3600_h24_d128.md",
    ("k_attn_bf16", 2, "virtual"): "k_attn_bf16_virtual_hunyuanvideo_33x3600_h24_d128.md",
    ("k_attn_bf16", 3, "explicit"): "k_attn_bf16_hunyuanvideo_text_33x3600_t256_h24_d128.md",
    ("k_attn_bf16", 4, "explicit"): "k_attn_bf16_sparse_vdit_21x1560_h40_d128.md",
    ("k_attn_fp8", 2, "virtual"): "k_attn_fp8_hunyuanvideo_33x3600_h24_d128.md",
    ("k_attn_fp8pv", 2, "virtual"): "k_attn_fp8pv_hunyuanvideo_33x3600_h24_d128.md",
}


def source_sha256(kernel):
    """sha256 over the sources of a timed kernel (k_attn_fp8pv is built from
    the k_attn_fp8 file)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES["k_attn_fp8" if kernel == "k_attn_fp8pv" else kernel]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def read_record(path):
    """The '- key: value' lines of a summary's record block."""
    rec = {}
    for line in open(path).read().splitlines():
        if line.startswith("- record_"):
            k, _, v = line[2:].partition(":")
            rec[k.strip()] = v.strip()
    return rec


def recorded_traffic(kernel, config, layout):
    """HBM bytes per dispatch of the timed kernel from the committed rocprofv3
    counter summary of this workload and layout (FETCH_SIZE + WRITE_SIZE,
    calibrated), or None when there is none or the kernel's sources have
    changed since the counters were taken."""
    name = TRAFFIC_RECORDS.get((kernel, config, layout))
    if name is None:
        return None
    try:
        rec = read_record(os.path.join(ROOT, "profiles", name))
        sha = source_sha256(kernel)
    except OSError:
        return None
    if rec.get("record_source_sha256") != sha or rec.get("record_kernel") != kernel or \
            "record_traffic_bytes_per_dispatch" not in rec:
        return None
    return float(rec["record_traffic_bytes_per_dispatch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, inp, labels, d, scale, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    masked attention of seeded query rows of two heads (one per label kind
    present), timed on the host cores; reported in TFLOP/s of the same
    4*d*pairs accounting."""
    import numpy as np

    import oracle
    c = cfg
    og = oracle.geom(c["N"], c["F"], c["T"], c["a1"], c["a2"], c.get("window", c["F"]), c.get("stripe", 512))
    heads = []
    for want in sorted(set(int(x) for x in labels)):
        if want == 3:
            continue
        heads.append(int(np.nonzero(labels == want)[0][0]))
    heads = heads[:2]
    rng = np.random.default_rng(99)
    L = c["T"] + c["N"] * c["F"]
    seen = {}

    def keys_of(mode, r):  # active keys of row r under mode (memoised: rows repeat on small shapes)
        if (mode, r) not in seen:
            seen[(mode, r)] = sum(hi - lo for lo, hi in oracle.row_intervals(og, mode, r))
        return seen[(mode, r)]

    flops = 0.0
    elapsed = 0.0
    rows_done = 0
    n = 8
    while elapsed < budget_s:
        m = min(n, L)
        for h in heads:
            rows = np.sort(rng.choice(L, size=m, replace=False)).astype(np.int64)
            t0 = time.perf_counter()
            oracle.attention_rows(og, int(labels[h]), inp["q"][h], inp["k"][h], inp["v"][h], scale, rows)
            elapsed += time.perf_counter() - t0
            mode = oracle.TEMPORAL if labels[h] == 1 else int(labels[h])
            for r in rows:
                flops += 4.0 * d * keys_of(mode, int(r))
            rows_done += m
        n = min(2 * n, 2048)
    out = {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{rows_done} seeded query rows of heads {heads} (labels "
                     f"{[int(labels[h]) for h in heads]}), fp64 oracle masked attention, {elapsed:.1f} s",
           "cpu_model": cpu_model()}
    if inp["rows"] is not None:
        # the oracle's profiling of one head on the layer's sampled rows (full,
        # spatial and temporal attention of those rows), same accounting
        rows = inp["rows"].astype(np.int64)
        t0 = time.perf_counter()
        oracle.profile_head(og, inp["q"][0], inp["k"][0], inp["v"][0], scale, rows)
        pt = time.perf_counter() - t0
        pflops = 0.0
        for mode in (oracle.FULL, oracle.SPATIAL, oracle.TEMPORAL):
            for r in rows:
                pflops += 4.0 * d * keys_of(mode, int(r))
        out["profile_value"] = pflops / pt / 1e12
        out["profile_sample"] = f"oracle profiling of head 0 on its {rows.size} sampled rows, {pt:.1f} s"
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def search_keys(geom, rows):
    """Keys per sampled row summed over the four masks the mode search sweeps
    (full, window, temporal band, stripe), from the masks' closed forms."""
    import numpy as np
    N, F, T = geom.N, geom.F, geom.T
    n = N * F
    u = rows.astype(np.int64) - T
    j = u % F
    full = T + n
    window = T + np.minimum(u + geom.window, n) - np.maximum(u - geom.window + 1, 0)
    temporal = T + N * (np.minimum(F, j + geom.a2) - np.maximum(0, j - geom.a2 + 1))
    stripe = T + min(geom.stripe, n)
    return float(np.sum(full + window + temporal + stripe))


def time_search(args, svg, S, geom, q, k, v, inp, dev, np, torch):
    rows_np = inp["rows"]
    if rows_np is None:
        rows_np = S.sample_rows(geom.N, geom.F, geom.T, 0.01, inp["seed"] + 500)
    rows = torch.from_numpy(rows_np.astype(np.int32)).to(dev)
    ws = svg.alloc_workspace(geom, svg.BF16, rows.numel(), svg.MODE_SEARCH | svg.VIRTUAL_PERMUTE)
    modes = torch.empty(geom.B * geom.H, dtype=torch.int32, device=dev)
    stats = torch.empty(geom.B * geom.H * 8, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        svg.svg_search_modes(geom, q, k, v, rows, modes, stats, ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        svg.svg_search_modes(geom, q, k, v, rows, modes, stats, ws)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = 4.0 * geom.d * geom.B * geom.H * search_keys(geom, rows_np)
    m = modes.cpu().numpy()
    names = {svg.FULL: "full", svg.SKIP: "skip", svg.WINDOW: "window", svg.TEMPORAL: "temporal",
             svg.STRIPE: "stripe"}
    log(f"mode search: {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    return {"search_ms": round(ms, 4), "search_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "search_rows": int(rows_np.size), "search_lambda": 0.5, "search_eps": 1.0,
            "search_modes": {nm: int((m == c).sum()) for c, nm in names.items()}}


def time_svg2(args, svg, S, cfg, dev, np, torch):
    """svg2_forward (k-means of Q and K from the strided start, selection,
    K/V gather, attention) on SVG2-shaped inputs of the same geometry: 256
    planted semantic groups per head, C_q = C_k = 256, 3 Lloyd iterations,
    p = 0.9."""
    C, iters, p = 256, 3, 0.9
    g = svg.Geom(B=1, H=cfg["H"], d=cfg["d"], N=cfg["N"], F=cfg["F"], T=cfg["T"])
    H, d, L = g.H, g.d, g.L
    t0 = time.time()
    inp = S.svg2_inputs(g.N, g.F, g.T, H, d, C, seed=31, spread=args.svg2_spread)
    log(f"svg2 inputs generated in {time.time() - t0:.1f} s")
    q, k, v = (torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16)[None] for n in "qkv")
    del inp
    o = torch.empty_like(q)
    prm = svg.Svg2Params(C, C, iters, p)
    mq = torch.empty(H * C * d, dtype=torch.float32, device=dev)
    mk = torch.empty_like(mq)
    sel = torch.empty(H * C * C, dtype=torch.uint8, device=dev)
    ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device=dev)
    lab = torch.empty(H * L, dtype=torch.int32, device=dev)
    perm = torch.empty_like(lab)
    start = torch.empty(H * (C + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    fwd_ms = timed(lambda: svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel))
    log(f"svg2 forward: {fwd_ms:.3f} ms")
    counts = []
    for x in (q, k):
        svg.svg2_kmeans(g, x, C, iters, mq, lab, perm, start, ws)
        st = start.cpu().numpy().reshape(H, C + 1)
        counts.append(np.diff(st, axis=1).astype(np.float64))
    km_ms = timed(lambda: (svg.svg2_kmeans(g, q, C, iters, mq, lab, perm, start, ws),
                           svg.svg2_kmeans(g, k, C, iters, mk, lab, perm, start, ws)))
    sl = sel.cpu().numpy().reshape(H, C, C).astype(np.float64)
    pairs = float(np.einsum("ha,hab,hb->", counts[0], sl, counts[1]))
    flops = 4.0 * d * pairs
    rest_ms = fwd_ms - km_ms
    log(f"svg2 k-means (Q and K): {km_ms:.3f} ms, density {pairs / (H * L * L):.4f}")
    return {"svg2_ms": round(fwd_ms, 4), "svg2_kmeans_ms": round(km_ms, 4),
            "svg2_select_gather_attn_ms": round(rest_ms, 4),
            "svg2_density": round(pairs / (H * L * L), 4),
            "svg2_effective_tflops": round(flops / (fwd_ms * 1e-3) / 1e12, 2),
            "svg2_attn_tflops_est": round(flops / (rest_ms * 1e-3) / 1e12, 2) if rest_ms > 0 else None,
            "svg2_config": {"clusters_q": C, "clusters_k": C, "iters": iters, "p": p, "init": "strided",
                            "planted_groups": C, "spread": args.svg2_spread, "noise": 0.3}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", "--config", dest="config", type=int, default=2,
                    help="synthetic workload: 0 tiny fp32 4x64, 1 CogVideoX-shaped 13x4080 h48 d64, "
                         "2 HunyuanVideo-shaped 33x3600 h24 d128 (default), 3 the same with 256 text tokens and "
                         "mixed heads, 4 Sparse-vDiT pattern set 21x1560 h40 d128")
    ap.add_argument("--call", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--virtual", action="store_true",
                    help="temporal heads gather through the index map instead of explicit permutes")
    ap.add_argument("--one-layout", action="store_true",
                    help="time only the headline layout (profiler runs: both layouts launch the same kernels)")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--search", action="store_true", help="also time svg_search_modes on the same inputs")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 E4M3 scores: quantise Q, K (svg_quantize_qk) and run svg_sparse_attention_fp8")
    ap.add_argument("--fp8-pv", action="store_true",
                    help="FP8 scores and FP8 P.V: svg_quantize_qk + svg_quantize_v + svg_sparse_attention_fp8_pv")
    ap.add_argument("--svg2", action="store_true",
                    help="also time svg2_forward (SVG2 semantic-aware permutation) on the same geometry")
    ap.add_argument("--svg2-spread", type=float, default=1.0, help="spread of the planted SVG2 group centres")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this path shards by head with no "
              "cross-GPU exchange, and multi-GPU measurement is not implemented here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_video_svg_amd as svg
    import svg_synth as S

    cfg = S.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = S.make_inputs(args.config, call=args.call)
    log(f"inputs for workload {args.config} ({cfg['name']}) generated in {time.time() - t0:.1f} s")
    bf16 = cfg["dtype"] == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    din = svg.BF16 if bf16 else svg.F32
    geom = svg.Geom(B=1, H=cfg["H"], d=cfg["d"], N=cfg["N"], F=cfg["F"], T=cfg["T"], a1=cfg["a1"], a2=cfg["a2"],
                    window=cfg.get("window", cfg["F"]), stripe=cfg.get("stripe", 512))
    H, d, L = geom.H, geom.d, geom.L
    q = torch.from_numpy(inp["q"]).to(dev).to(tdt)[None]
    k = torch.from_numpy(inp["k"]).to(dev).to(tdt)[None]
    v = torch.from_numpy(inp["v"]).to(dev).to(tdt)[None]
    o = torch.empty_like(q)
    profile = inp["rows"] is not None
    rows = torch.from_numpy(inp["rows"]).to(dev) if profile else None
    n_rows = 0 if rows is None else rows.numel()
    BM, BN = svg.svg_tile_config(din, d)
    nQT = -(-L // BM)
    labels = torch.empty(H, dtype=torch.int32, device=dev)
    stats = torch.empty(H * 3, dtype=torch.float32, device=dev)
    ranges = torch.empty(H * nQT * 4, dtype=torch.int32, device=dev)
    order = torch.empty(H, dtype=torch.int32, device=dev)
    ws = svg.alloc_workspace(geom, din, n_rows, svg.VIRTUAL_PERMUTE)
    if args.fp8_pv:
        args.fp8 = True
    if args.fp8:
        if not bf16:
            sys.exit("--fp8 needs a bf16 workload")
        args.virtual = True  # the fp8 path reads temporal heads through the index map
        nkt = -(-L // 64)
        q8 = torch.empty(H * L * d, dtype=torch.uint8, device=dev)
        k8 = torch.empty_like(q8)
        sq = torch.empty(H * L, dtype=torch.float32, device=dev)
        sk = torch.empty(H * nkt, dtype=torch.float32, device=dev)
        if args.fp8_pv:
            v8 = torch.empty(H * nkt * d * 64, dtype=torch.uint8, device=dev)
            svh = torch.empty(H, dtype=torch.float32, device=dev)
    modes_fixed = None if profile else torch.from_numpy(inp["kinds"].astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed_layer(virtual):
        """Warmup, then args.steps timed layers with temporal heads through
        explicit permuted copies (virtual False) or the index map (True).
        Returns (ms per step, per-stage ms means [profile, blocks, permute of
        K and V or quantise, attention, (empty)], wall ms per step)."""
        flags = svg.VIRTUAL_PERMUTE if virtual else 0
        # explicit layout: token-major copies of K and V (the attention kernel
        # reads Q and writes O of temporal heads through the index map)
        if not virtual:
            kp, vp = (torch.empty_like(t) for t in (k, v))
        else:
            kp = vp = None

        def step(marks):
            """One layer; records an event after each stage into marks (list)."""
            marks.append(ev()); marks[-1].record(stream)
            if profile:
                svg.svg_profile_heads(geom, q, k, v, rows, labels, stats, ws)
                modes = labels
            else:
                modes = modes_fixed
            marks.append(ev()); marks[-1].record(stream)
            svg.svg_build_blocks(geom, modes, BM, BN, ranges, order)
            marks.append(ev()); marks[-1].record(stream)
            if args.fp8:
                svg.svg_quantize_qk(geom, q, k, modes, q8, sq, k8, sk)
                if args.fp8_pv:
                    svg.svg_quantize_v(geom, v, modes, v8, svh)
            elif not virtual:
                for s_, d_ in ((k, kp), (v, vp)):
                    svg.svg_layout_permute(geom, s_, d_, modes=modes)
            marks.append(ev()); marks[-1].record(stream)
            if args.fp8_pv:
                svg.svg_sparse_attention_fp8_pv(geom, q8, sq, k8, sk, v8, svh, o, modes, ranges, order)
            elif args.fp8:
                svg.svg_sparse_attention_fp8(geom, q8, sq, k8, sk, v, o, modes, ranges, order)
            else:
                svg.svg_sparse_attention(geom, q, k, v, o, modes, ranges, order, kp=kp, vp=vp, flags=flags)
            marks.append(ev()); marks[-1].record(stream)
            # (no inverse permute: temporal heads' outputs are written in place)
            marks.append(ev()); marks[-1].record(stream)

        for i in range(args.warmup):
            step([])
        torch.cuda.synchronize()
        log(f"warmup done ({args.warmup} steps, {'virtual' if virtual else 'explicit'} layout)")
        all_marks = []
        start, end = ev(), ev()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            m = []
            step(m)
            all_marks.append(m)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms = start.elapsed_time(end) / args.steps
        stage = np.array([[m[j].elapsed_time(m[j + 1]) for j in range(5)] for m in all_marks]).mean(axis=0)
        log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f})")
        return ms, stage, wall * 1e3 / args.steps

    ms_per_step, stage, _ = timed_layer(args.virtual)
    prof_ms, blocks_ms, perm_ms, attn_ms, _ = stage
    # the other layout of the same layer (bit-identical outputs), reported beside it
    alt = None
    if not args.fp8 and not args.one_layout:
        alt_ms, alt_stage, _ = timed_layer(not args.virtual)
        alt = (not args.virtual, alt_ms, alt_stage)

    # a4 on its own: every head of Q through the layout transformation (one
    # [B, H, L, d] tensor read and written), timed apart from the step
    qa = torch.empty_like(q)
    for _ in range(2):
        svg.svg_layout_permute(geom, q, qa)
    pa, pb = ev(), ev()
    pa.record(stream)
    for _ in range(5):
        svg.svg_layout_permute(geom, q, qa)
    pb.record(stream)
    torch.cuda.synchronize()
    perm_all_ms = pa.elapsed_time(pb) / 5
    perm_all_gbs = 2.0 * q.numel() * q.element_size() / (perm_all_ms * 1e-3) / 1e9
    # a6 on its own as well (the layer writes temporal heads' outputs in
    # place through the index map instead): the inverse of the whole tensor
    qb = torch.empty_like(q)
    for _ in range(2):
        svg.svg_layout_permute(geom, qa, qb, inverse=True)
    pa.record(stream)
    for _ in range(5):
        svg.svg_layout_permute(geom, qa, qb, inverse=True)
    pb.record(stream)
    torch.cuda.synchronize()
    inv_all_ms = pa.elapsed_time(pb) / 5
    inv_all_gbs = 2.0 * q.numel() * q.element_size() / (inv_all_ms * 1e-3) / 1e9
    del qa, qb

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    lab = labels.cpu().numpy() if profile else inp["kinds"].astype(np.int32)
    pairs = [pair_count(geom.N, geom.F, geom.T, int(m), geom.a1, geom.a2, geom.window, geom.stripe) for m in lab]
    flops = 4.0 * d * float(sum(pairs))
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = ((PEAK_FP8_TFLOPS if args.fp8_pv else PEAK_FP8_QK_TFLOPS) if args.fp8 else PEAK_BF16_TFLOPS) \
        if bf16 else PEAK_F32_TFLOPS
    n_temporal = int((lab == 1).sum())
    elt = 2 if bf16 else 4
    perm_bytes = 2.0 * n_temporal * L * d * elt  # read + write per permuted head-tensor
    explicit = not args.virtual and n_temporal
    fwd_gbs = 2 * perm_bytes / (perm_ms * 1e-3) / 1e9 if explicit and perm_ms > 0 else None  # K and V
    timed_kernel = "k_attn_fp8pv" if args.fp8_pv else "k_attn_fp8" if args.fp8 else "k_attn_bf16"
    result = {
        "metric": "sparse-attn ms/layer + effective TFLOP/s vs bf16 MFMA peak (33x3600x24h x d128)",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded planted Q/K/V, no model activations)",
        "config": {"workload": cfg["name"], "frames": geom.N,
                   "tokens_per_frame": geom.F, "text_tokens": geom.T, "heads": H, "head_dim": d,
                   "a1": geom.a1, "a2": geom.a2, "sampled_rows": n_rows, "layout": "virtual" if args.virtual
                   else "explicit", "scores": "fp8-e4m3 (Q per row, K per 64-key tile)" if args.fp8 else "bf16",
                   "pv": "fp8-e4m3 (P in-kernel, V per head)" if args.fp8_pv else "bf16",
                   "labels": {"spatial": int((lab == 0).sum()), "temporal": n_temporal,
                                               "full": int((lab == 2).sum()), "other": int((lab > 2).sum())}},
        "attn_ms": round(float(attn_ms), 4),
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_of_peak": round(attn_tflops / peak, 4),
        "profile_ms": round(float(prof_ms), 4),
        "blocks_ms": round(float(blocks_ms), 4),
        "permute_fwd_ms": None if args.fp8 else round(float(perm_ms), 4),
        "quant_ms": round(float(perm_ms), 4) if args.fp8 else None,
        "permute_fwd_gbs": None if fwd_gbs is None else round(fwd_gbs, 1),
        "permute_all_heads_ms": round(perm_all_ms, 4),
        "permute_all_heads_gbs": round(perm_all_gbs, 1),
        "permute_all_heads_frac_of_hbm": round(perm_all_gbs / 8000.0, 4),
        "permute_inverse_all_heads_ms": round(inv_all_ms, 4),
        "permute_inverse_all_heads_gbs": round(inv_all_gbs, 1),
        "effective_flops_per_layer": flops,
        "other_layout": None if alt is None else {
            "layout": "virtual" if alt[0] else "explicit",
            "value": round(flops / (alt[1] * 1e-3) / 1e12, 2), "ms_per_step": round(alt[1], 4),
            "attn_ms": round(float(alt[2][3]), 4), "attn_frac_of_peak": round(flops / (alt[2][3] * 1e-3) / 1e12 / peak, 4),
            "profile_ms": round(float(alt[2][0]), 4),
            "permute_fwd_ms": round(float(alt[2][2]), 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4),
                     "traffic": recorded_traffic(timed_kernel, args.config,
                                                 "virtual" if args.virtual else "explicit") if bf16 else None,
                     "kernel": ("k_attn_fp8<PV8> (svg_sparse_attention_fp8_pv)" if args.fp8_pv else
                                "k_attn_fp8 (svg_sparse_attention_fp8)" if args.fp8 else
                                "k_attn_bf16 (svg_sparse_attention)") if bf16 else "k_attn_f32"},
    }
    if args.search and bf16:
        result.update(time_search(args, svg, S, geom, q, k, v, inp, dev, np, torch))
    if args.svg2 and bf16:
        result.update(time_svg2(args, svg, S, cfg, dev, np, torch))
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, lab, d, 1.0 / np.sqrt(d))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
