"""Dual-flow grouped decode benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c5|c3|c4]

A step is one grouped decode step of the whole model (every layer, the LM
head and the mixture head) for all B sequences, both flows. Inputs are seeded
synthetic tensors of the workload's shapes, already resident in HBM when the
timed region starts; each step decodes greedily from the previous step's
mixture argmax, so the context grows by one position per step. Prints one
JSON line: decode tokens/s, the roofline of the dominant kernel (the
shared-K/V attention pass, timed with HIP events on its stream), the
whole-step achieved bandwidth, the dual/primary byte and time ratios, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dual-flow decode tokens/s at 1 GPU; achieved HBM GB/s vs peak; dual/primary byte ratio"
PEAK_HBM_GBS = 8000.0
# Decode attention launches timed inside the timed region: one in every 7 (a timed launch takes a
# few microseconds more than an untimed one; 7 shares no factor with 16, 24 or 32 layers, so the
# sample walks through every layer).
TIMING_STRIDE = 7

# HBM traffic measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (one pass each, 1 warm-up + 2
# timed steps, dual and primary-only), counters scaled by their reading for a plain 1 GiB copy
# (x2.0 fetch, x1.0 write). Reported only while the kernel sources are the ones they were
# measured on (attention pass: attention.hip; step traffic: every library source).
COUNTER_SOURCES = {"attention_source_sha256": "b5eb70e54b8ee2d865fa1c741f1b650fdb21be0a0a533d09e4075cd9f5bf56e9",
                   "library_sources_sha256": "5d2586b0f473afd81e105517cdd486b3ab82bd3295804fe83514d7c94db9e556"}
COUNTERS = {
    "dense_32l_d4096_b16_ctx8192": {"attention_traffic_bytes_per_launch": 2.15500e+09,
                   "step_traffic_bytes": {"dual": 8.39800e+10, "primary_only": 8.29850e+10}},
    "dense_1p3b_b16_ctx2048": {"attention_traffic_bytes_per_launch": 2.73400e+08,
                   "step_traffic_bytes": {"dual": 9.89500e+09, "primary_only": 9.47300e+09}},
    "moe_16l_e64_top4_b64_ctx1024": {"attention_traffic_bytes_per_launch": 5.47600e+08,
                   "step_traffic_bytes": {"dual": 1.93000e+10, "primary_only": 1.85690e+10}},
}


def source_hashes():
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "dual_flow_transformer_amd", "csrc")
    att = hashlib.sha256(open(os.path.join(csrc, "attention.hip"), "rb").read()).hexdigest()
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(open(f, "rb").read())
    return att, h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=["c2", "c3", "c4", "c5", "prefill", "forward"],
                    help="c5 (default) / c3 / c4: full decode step; c2: the shared-K/V attention kernel alone; "
                         "prefill: primary prefill of 16 x 2048 tokens through the 1.3B dense model; "
                         "forward: full-sequence dual forward of the same model and tokens")
    ap.add_argument("--variant", type=int, default=0,
                    help="model variant switches: 1 couplings off, 2 aux output (no mixture), 4 alpha=(1+CP)/2")
    ap.add_argument("--top-k-aux", type=int, default=0,
                    help="MoE: aux expert fan-out from the primary ranking (0 = replay of top_k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-primary-pass", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=0, help="oracle sample: layers (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--primary-only", action="store_true",
                    help="time primary-only steps instead of dual steps (byte-ratio profiling)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stream_read_ceiling(buf, attn_bytes: float, attn_gbs: float, stream) -> dict:
    """The practical read rate of the device in the attention pass's launch
    shape: df_stream_read (one 4-wave workgroup per CU, contiguous share per
    wave, 16-byte non-temporal loads) over the first bytes of `buf` (the K
    cache), 10 back-to-back calls per size. Sizes 8 MiB .. 512 MiB give the
    fixed cost per launch and the streaming rate (least squares of time =
    fixed + bytes / rate); one size equals the attention pass's bytes per
    launch, whose rate the attention's is compared with."""
    import numpy as np
    import torch

    from dual_flow_transformer_amd import _abi

    have = buf.numel() * buf.element_size()
    out = torch.zeros(_abi.DF_STREAM_READ_OUT_WORDS, dtype=torch.int32, device="cuda")
    att = int(attn_bytes) // 16 * 16
    sizes = [n for n in (8 << 20, 32 << 20, 128 << 20, 512 << 20) if n <= have]
    rows = []
    for n in sizes + ([att] if att <= have else []):
        call = lambda: _abi.check(_abi.df_stream_read(buf.data_ptr(), n, out.data_ptr(), stream.cuda_stream),
                                  "df_stream_read")
        call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        rows.append((n, e0.elapsed_time(e1) * 1e3 / 10))
    res = {"kernel": "df_stream_read", "calls_per_size": 10,
           "bytes": [r[0] for r in rows], "us_per_call": [round(r[1], 2) for r in rows]}
    if len(sizes) >= 2:
        x = np.array([r[0] for r in rows[:len(sizes)]], dtype=np.float64)
        y = np.array([r[1] for r in rows[:len(sizes)]], dtype=np.float64)
        slope, fixed = np.polyfit(x, y, 1)
        res["fit_fixed_us"] = float(fixed)
        res["fit_streaming_GBs"] = float(1e-3 / slope)
    if att <= have:
        read_gbs = att / rows[-1][1] / 1e3
        res["attention_bytes_GBs"] = read_gbs
        res["attention_frac_of_read"] = attn_gbs / read_gbs
        log(f"[bench] streaming read of the attention's {att / 1e9:.3f} GB: {rows[-1][1]:.1f} us "
            f"({read_gbs:.0f} GB/s); attention pass at {attn_gbs / read_gbs:.3f} of it")
    return res


def cpu_baseline(cfg, n_layers: int, min_seconds: float = 10.0):
    """The CPU oracle as it stands, on a bounded sample: sequence 0 of the
    workload through its first n_layers layers plus the LM head and mixture
    head (inputs drawn and decoded before timing), repeated until at least
    min_seconds of CPU work. Per-token time = layers scaled to the full depth
    + head; value = tokens/s of one oracle instance."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dualflow as odf
    from synth.workloads import Inputs

    sub = cfg.replace(L=n_layers)
    src = Inputs(sub)
    model = odf.Model(src, keep_layers=True)
    for l in range(n_layers):
        model.layer(l)
    model.w_out()
    model.lnf()
    cache = odf.Cache(sub, [0], src)
    for l in range(n_layers):
        cache.layer(l)
    rl = None
    if cfg.moe:
        rl = np.stack([src.router_logits(0, l)[:1] for l in range(n_layers)])
    tok = src.step_tokens(0)[:1]
    # time the layers and the head separately: full-depth extrapolation
    t_total, reps, t_head = 0.0, 0, 0.0
    while t_total < min_seconds or reps < 1:
        cache.lens[:] = cfg.ctx          # every repetition is the same step
        t0 = time.perf_counter()
        r = odf.decode_step(model, cache, tok, aux_on=True, router_logits=rl)
        t_total += time.perf_counter() - t0
        reps += 1
    h = np.zeros((1, 2, cfg.d))
    t0 = time.perf_counter()
    for i in range(reps):
        for f in range(2):
            odf._matvec(model.w_out(), odf.round_to(odf.layer_norm(h[0, f], model.lnf(), cfg.eps), cfg.dtype))
        odf.mix_head(np.zeros(cfg.V), np.zeros(cfg.V))
    t_head = (time.perf_counter() - t0) / reps
    t_step = t_total / reps
    t_layer = max(t_step - t_head, 1e-9) / n_layers
    t_tok = t_layer * cfg.L + t_head
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": 1.0 / t_tok, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"sequence 0 of {cfg.B}, first {n_layers} of {cfg.L} layers + LM head + mixture head, "
                       f"{reps} steps ({t_total:.1f} s); per-token time scaled to {cfg.L} layers"),
            "seconds_per_token": t_tok, "host_cpus": os.cpu_count()}


def bench_attention(args):
    """Attention-only workload: batch 32, 32 heads x 128, lengths uniform in
    [1024, 4096], bf16 K/V, two queries per head. Times K calls of
    df_attention_dual (partial pass + combine) after W warm-up calls; the
    value is the achieved HBM bandwidth of the whole call over the algorithmic
    bytes (every K/V byte of the attended positions once, queries, outputs)."""
    import numpy as np
    import torch

    from dual_flow_transformer_amd import _abi
    from synth import device as synth_dev
    from synth import stream_id
    from synth.workloads import C2_ATTN, AttnInputs

    c = C2_ATTN
    src = AttnInputs(c)
    lens = src.lengths()
    log(f"[bench] attention workload {c.name}: lengths {lens.min()}..{lens.max()}")
    K_ = torch.empty((c.B, c.H, c.S_max, c.Dh), dtype=torch.int16, device="cuda")
    V_ = torch.empty_like(K_)
    for which, t in (("k", K_), ("v", V_)):
        st = [stream_id("attn_" + which, b, h) for b in range(c.B) for h in range(c.H)]
        synth_dev.normal_streams(t, st, c.S_max * c.Dh, c.S_max * c.Dh, c.seed, 1.0, True)
    q1, q2, a = src.queries()
    dq = torch.from_numpy(np.stack([q1, q2], axis=1)).cuda()
    da = torch.from_numpy(a).cuda()
    dl = torch.from_numpy(lens.astype(np.int32)).cuda()
    o = torch.empty((c.B, 2, c.H, c.Dh), device="cuda")
    lse = torch.empty((c.B, 2, c.H), device="cuda")
    wsb = _abi.df_attention_workspace_bytes(c.B, c.H, c.S_max, c.Dh)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        _abi.check(_abi.df_attention_dual(_abi.DF_BF16, K_.data_ptr(), V_.data_ptr(), c.B, c.H, c.S_max, c.Dh,
                                          dl.data_ptr(), dq.data_ptr(), da.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                          ws.data_ptr(), wsb, stream.cuda_stream), "df_attention_dual")

    W, K = args.warmup, args.steps
    for _ in range(W):
        call()
    torch.cuda.synchronize()
    _abi.check(_abi.df_timing_enable(0, TIMING_STRIDE), "df_timing_enable")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    rc, part_ms, part_n = _abi.df_timing_read()
    _abi.check(rc, "df_timing_read")
    ms = e0.elapsed_time(e1) / K
    kv_bytes = int(lens.astype(np.int64).sum()) * c.H * c.Dh * 2 * 2
    io_bytes = c.B * c.H * c.Dh * 4 * 2 * 2 + c.H * c.Dh * 4 + c.B * 2 * c.H * 4
    gbs = (kv_bytes + io_bytes) / (ms / 1e3) / 1e9
    part_avg = part_ms / max(part_n, 1)
    part_gbs = kv_bytes / (part_avg / 1e3) / 1e9
    log(f"[bench] attention call {ms * 1e3:.1f} us ({gbs:.0f} GB/s); partial pass {part_avg * 1e3:.1f} us")

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import dualflow as odf
        b = 0
        Kb = odf.to_f64(src.kv_block("k", b, int(lens[b])))
        Vb = odf.to_f64(src.kv_block("v", b, int(lens[b])))
        t, reps = 0.0, 0
        while t < 10.0:
            t0 = time.perf_counter()
            for h in range(c.H):
                qq2 = q2[b, h] + a.reshape(c.H, c.Dh)[h] * q1[b, h]
                for qq in (q1[b, h], qq2):
                    odf.attention_one(qq.astype(np.float64), Kb[h], Vb[h])
            t += time.perf_counter() - t0
            reps += 1
        per_seq = t / reps
        seq_bytes = int(lens[b]) * c.H * c.Dh * 2 * 2
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": seq_bytes / per_seq / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
               "sample": f"sequence 0 ({int(lens[b])} positions, all {c.H} heads, both queries), {reps} repetitions "
                         f"({t:.1f} s)", "seconds_per_call_scaled": per_seq * float(lens.sum()) / float(lens[b])}
    out = {
        "metric": "shared-K/V dual-query attention: achieved HBM GB/s vs peak", "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded K/V and queries)",
        "config": {"workload": c.name, "batch": c.B, "heads": c.H, "head_dim": c.Dh,
                   "lengths": [int(lens.min()), int(lens.max())], "mean_length": float(lens.mean())},
        "roofline": {"kernel": "attn_partial (split-K pass)", "bound": "hbm", "achieved": part_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": part_gbs / PEAK_HBM_GBS, "traffic": None,
                     "avg_launch_ms": part_avg, "launches": part_n, "timed_every": TIMING_STRIDE,
                     "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


PEAK_BF16_TFLOPS = 2500.0


def prefill_flops(cfg, T: int) -> dict:
    """Algorithmic flops of a primary prefill of T positions per sequence from
    an empty cache: 2 flops per multiply-add of every projection row (QKV, O,
    up, down) and of the causal attention (scores and weighted values over
    keys 0..t for position t)."""
    proj = 2 * cfg.B * T * (4 * cfg.d * cfg.d + 2 * cfg.d * cfg.F) * cfg.L
    attn = 2 * 2 * cfg.B * cfg.d * (T * (T + 1) // 2) * cfg.L
    return {"projections": proj, "attention": attn, "total": proj + attn}


def prefill_cpu_baseline(cfg, T: int, n_layers: int = 1, min_seconds: float = 10.0):
    """The oracle's prefill as it stands on a bounded sample: sequence 0's
    prompt through the first n_layers layers (inputs drawn before timing),
    repeated until min_seconds; tokens/s scaled to the full depth."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dualflow as odf
    from synth.workloads import Inputs

    sub = cfg.replace(L=n_layers, B=1)
    src = Inputs(sub)
    model = odf.Model(src, keep_layers=True)
    for l in range(n_layers):
        model.layer(l)
    model.w_out()
    model.lnf()
    prompt = Inputs(cfg).prompt()[:1, :T]
    t, reps = 0.0, 0
    while t < min_seconds or reps < 1:
        cache = odf.Cache(sub, [0], src)
        cache.lens[:] = 0
        t0 = time.perf_counter()
        odf.prefill_primary(model, cache, prompt)
        t += time.perf_counter() - t0
        reps += 1
    # the oracle also forms the logits of every prompt position; the GPU
    # prefill does not, so that part is timed alone and taken out
    h = np.zeros((T, cfg.d))
    t0 = time.perf_counter()
    odf.layer_norm(h, model.lnf(), cfg.eps) @ model.w_out().T
    t_head = time.perf_counter() - t0
    per_layer = max(t / reps - t_head, 1e-9) / n_layers
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": T / (per_layer * cfg.L), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"sequence 0 of {cfg.B}: its {T}-token prompt through the first {n_layers} of {cfg.L} "
                       f"layers, {reps} repetitions ({t:.1f} s, less {t_head:.1f} s per repetition for the "
                       f"logits of every position); time scaled to {cfg.L} layers"), "host_cpus": os.cpu_count()}


def bench_prefill(args):
    """Primary prefill workload: 16 prompts of 2048 tokens through the 24-layer
    d 2048 dense model (bf16 weights), empty cache. A step is one
    df_prefill_primary call over all prompts (len reset to 0 before it). The
    value is prompt tokens/s; the roofline is that of the tiled GEMM (the
    projections), timed with HIP events on its stream, against the dense
    bf16 matrix-core peak."""
    import torch

    from dual_flow_transformer_amd import _abi
    from dual_flow_transformer_amd.runtime import DecodeModel
    from synth.workloads import PREFILL_DENSE, Inputs

    cfg = PREFILL_DENSE
    T = cfg.prompt_len
    log(f"[bench] prefill workload {cfg.name}: filling device inputs")
    gm = DecodeModel(cfg, fill="device")
    tok = gm.tokens(Inputs(cfg).prompt()).contiguous()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        gm.len.zero_()
        gm.prefill(tok)

    W, K = args.warmup, args.steps
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    res = {}
    for kclass in (1, 2):              # GEMM launches, then attention launches, each over the K steps
        _abi.check(_abi.df_timing_enable(kclass, 1), "df_timing_enable")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        rc, kms, kn = _abi.df_timing_read()
        _abi.check(rc, "df_timing_read")
        res[kclass] = (e0.elapsed_time(e1) / K, kms, kn)
    ms = min(res[1][0], res[2][0])
    status = gm.status()
    fl = prefill_flops(cfg, T)
    tok_s = cfg.B * T / (ms / 1e3)
    gemm_ms, gemm_n = res[1][1], res[1][2]
    attn_ms, attn_n = res[2][1], res[2][2]
    gemm_tf = fl["projections"] / (gemm_ms / K / 1e3) / 1e12
    attn_tf = fl["attention"] / (attn_ms / K / 1e3) / 1e12
    log(f"[bench] prefill {ms:.2f} ms/step, {tok_s:.0f} tok/s; GEMM {gemm_ms / K:.2f} ms/step ({gemm_tf:.0f} TF/s), "
        f"attention {attn_ms / K:.2f} ms/step ({attn_tf:.0f} TF/s); status {status}")
    cpu = None
    if not args.no_cpu_baseline:
        del gm
        torch.cuda.empty_cache()
        cpu = prefill_cpu_baseline(cfg, T)
        log(f"[bench] oracle prefill: {cpu['value']:.2f} tok/s")
    out = {
        "metric": "primary prefill tokens/s at 1 GPU; GEMM TFLOP/s vs dense bf16 matrix-core peak",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights, uniform random prompt tokens)",
        "config": {"workload": cfg.name, "layers": cfg.L, "d_model": cfg.d, "heads": cfg.H, "head_dim": cfg.Dh,
                   "ffn": cfg.F, "global_batch": cfg.B, "prompt_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "gemm_bf16 (prefill projections)", "bound": "mfma", "achieved": gemm_tf,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": gemm_tf / PEAK_BF16_TFLOPS,
                     "traffic": None, "avg_launch_ms": gemm_ms / max(gemm_n, 1), "launches": gemm_n,
                     "algorithmic_flops_per_launch": fl["projections"] * K / max(gemm_n, 1)},
        "attention": {"kernel": "attn_prefill", "achieved_TFLOPs": attn_tf, "avg_launch_ms": attn_ms / max(attn_n, 1),
                      "launches": attn_n, "algorithmic_flops_per_step": fl["attention"]},
        "flops_per_step": fl, "device_status": status, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def forward_flops(cfg, T: int) -> dict:
    """Algorithmic flops of the dual forward of T positions per sequence from
    an empty cache: the primary flow as in the prefill; the aux flow's Q,
    O, up and down projections (its K/V columns are not formed); both
    flows' causal attention; the LM head of both flows at every position."""
    pri = prefill_flops(cfg, T)
    aux_proj = 2 * cfg.B * T * (2 * cfg.d * cfg.d + 2 * cfg.d * cfg.F) * cfg.L
    head = 2 * 2 * cfg.B * T * cfg.d * cfg.V
    proj = pri["projections"] + aux_proj + head
    attn = 2 * pri["attention"]
    return {"projections": proj, "attention": attn, "total": proj + attn}


def forward_cpu_baseline(cfg, T: int, n_layers: int = 1, min_seconds: float = 10.0):
    """The oracle's dual forward on a bounded sample: sequence 0's T tokens
    through the first n_layers layers plus the LM head and mixture of every
    position, repeated until min_seconds; the layer part scaled to full
    depth."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dualflow as odf
    from synth.workloads import Inputs

    sub = cfg.replace(L=n_layers, B=1)
    src = Inputs(sub)
    model = odf.Model(src, keep_layers=True)
    for l in range(n_layers):
        model.layer(l)
    model.w_out()
    model.lnf()
    toks = Inputs(cfg).prompt()[:1, :T]
    t, reps = 0.0, 0
    while t < min_seconds or reps < 1:
        cache = odf.Cache(sub, [0], src)
        cache.lens[:] = 0
        t0 = time.perf_counter()
        odf.forward_dual(model, cache, toks)
        t += time.perf_counter() - t0
        reps += 1
    # the head part (final norm, LM head of both flows, mixture per position) timed alone
    h = np.zeros((T, cfg.d))
    t0 = time.perf_counter()
    lg = [odf.layer_norm(h, model.lnf(), cfg.eps) @ model.w_out().T for _ in range(2)]
    for i in range(T):
        odf.mix_head(lg[0][i], lg[1][i])
    t_head = time.perf_counter() - t0
    t_tok = ((t / reps - t_head) / n_layers * cfg.L + t_head) / T
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": 1.0 / t_tok, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"sequence 0 of {cfg.B}: its {T} tokens through the first {n_layers} of {cfg.L} layers "
                       f"and the LM head + mixture of every position, {reps} repetitions ({t:.1f} s); layer time "
                       f"scaled to {cfg.L} layers"), "host_cpus": os.cpu_count()}


def bench_forward(args):
    """Dual forward workload: 16 sequences of 2048 tokens through the 24-layer
    d 2048 dense model, both flows at every position, empty cache. A step is
    one df_forward_dual call (len reset to 0 before it) producing p_mix and
    alpha of every position. Value: tokens/s (positions, both flows each);
    roofline: the tiled GEMM against the dense bf16 matrix-core peak."""
    import torch

    from dual_flow_transformer_amd import _abi
    from dual_flow_transformer_amd.runtime import DecodeModel
    from synth.workloads import FORWARD_DENSE, Inputs

    cfg = FORWARD_DENSE
    T = cfg.prompt_len
    log(f"[bench] forward workload {cfg.name}: filling device inputs")
    gm = DecodeModel(cfg, fill="device")
    tok = gm.tokens(Inputs(cfg).prompt()).contiguous()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        gm.len.zero_()
        gm.forward(tok, logits=False, next_tok=False)

    W, K = args.warmup, args.steps
    for _ in range(max(W, 1)):
        step()
    torch.cuda.synchronize()
    res = {}
    for kclass in (1, 2):
        _abi.check(_abi.df_timing_enable(kclass, 1), "df_timing_enable")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        rc, kms, kn = _abi.df_timing_read()
        _abi.check(rc, "df_timing_read")
        res[kclass] = (e0.elapsed_time(e1) / K, kms, kn)
    ms = min(res[1][0], res[2][0])
    status = gm.status()
    fl = forward_flops(cfg, T)
    tok_s = cfg.B * T / (ms / 1e3)
    gemm_ms, gemm_n = res[1][1], res[1][2]
    attn_ms, attn_n = res[2][1], res[2][2]
    gemm_tf = fl["projections"] / (gemm_ms / K / 1e3) / 1e12
    attn_tf = fl["attention"] / (attn_ms / K / 1e3) / 1e12
    log(f"[bench] forward {ms:.2f} ms/step, {tok_s:.0f} tok/s; GEMM {gemm_ms / K:.2f} ms/step ({gemm_tf:.0f} TF/s), "
        f"attention {attn_ms / K:.2f} ms/step ({attn_tf:.0f} TF/s); status {status}")
    cpu = None
    if not args.no_cpu_baseline:
        del gm
        torch.cuda.empty_cache()
        cpu = forward_cpu_baseline(cfg, T)
        log(f"[bench] oracle forward: {cpu['value']:.2f} tok/s")
    out = {
        "metric": "dual-flow full-sequence forward tokens/s at 1 GPU; GEMM TFLOP/s vs dense bf16 matrix-core peak",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights, uniform random tokens)",
        "config": {"workload": cfg.name, "layers": cfg.L, "d_model": cfg.d, "heads": cfg.H, "head_dim": cfg.Dh,
                   "ffn": cfg.F, "vocab": cfg.V, "global_batch": cfg.B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "gemm_bf16 (projections and LM head of both flows)", "bound": "mfma",
                     "achieved": gemm_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": gemm_tf / PEAK_BF16_TFLOPS,
                     "traffic": None, "avg_launch_ms": gemm_ms / max(gemm_n, 1), "launches": gemm_n,
                     "algorithmic_flops_per_launch": fl["projections"] * K / max(gemm_n, 1)},
        "attention": {"kernel": "attn_prefill (both query sets)", "achieved_TFLOPs": attn_tf,
                      "avg_launch_ms": attn_ms / max(attn_n, 1), "launches": attn_n,
                      "algorithmic_flops_per_step": fl["attention"]},
        "flops_per_step": fl, "device_status": status, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not part of "
              "this build. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "c2":
        bench_attention(args)
        return
    if args.workload == "prefill":
        bench_prefill(args)
        return
    if args.workload == "forward":
        bench_forward(args)
        return
    import numpy as np
    import torch

    from dual_flow_transformer_amd import _abi
    from dual_flow_transformer_amd.runtime import DecodeModel
    from synth.workloads import PRESETS, Inputs

    cfg = PRESETS[args.workload]
    W, K = args.warmup, args.steps
    S = cfg.ctx + W + K + 8
    cfg = cfg.replace(S_max=S, variant=args.variant, top_k_aux=args.top_k_aux if cfg.moe else 0)
    log(f"[bench] workload {cfg.name}: filling device inputs (S_max={S})")
    t0 = time.time()
    gm = DecodeModel(cfg, fill="device")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s; workspace {gm.ws_bytes / 2**20:.1f} MiB")
    src = Inputs(cfg)
    rls = None
    if cfg.moe:
        rls = [gm.router_logits(s) for s in range(W + K)]
    tok0 = gm.tokens(src.step_tokens(0))
    len0 = gm.len.clone()

    def run(n, first, aux_on=True):
        for i in range(n):
            s = first + i
            toks = tok0 if s == 0 else gm.next_tok
            gm.decode_step(toks, aux_on=aux_on,
                           router_logits=rls[s] if rls is not None else None, logits=False)

    stream = torch.cuda.current_stream()
    dual = not args.primary_only
    # warmup
    run(W, 0, aux_on=dual)
    torch.cuda.synchronize()
    lens_start = gm.len.cpu().numpy().astype(np.int64)
    # timed region: K dual steps
    _abi.check(_abi.df_timing_enable(0, TIMING_STRIDE), "df_timing_enable")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    run(K, W, aux_on=dual)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    rc, attn_ms, attn_n = _abi.df_timing_read()
    _abi.check(rc, "df_timing_read")
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / K
    tok_s = cfg.B * K / (ms / 1e3)
    status = gm.status()
    log(f"[bench] {K} steps: {ms_step:.3f} ms/step (wall {wall / K * 1e3:.3f}), {tok_s:.1f} tok/s, status {status}")

    # algorithmic bytes over the timed steps
    es = 2 if cfg.dtype == "bf16" else 4
    kv_attn = 0
    sampled = range(0, K * cfg.L, TIMING_STRIDE)          # the launches df_timing_enable timed
    assert len(sampled) == attn_n, (len(sampled), attn_n)
    for i in sampled:
        keys = int((lens_start + i // cfg.L + 1).sum())
        kv_attn += cfg.H * keys * cfg.Dh * es * 2
    attn_bytes_per_launch = kv_attn / len(sampled)
    attn_avg_ms = attn_ms / max(attn_n, 1)
    attn_gbs = attn_bytes_per_launch / (attn_avg_ms / 1e3) / 1e9
    gm.len.copy_(torch.from_numpy(lens_start + K // 2).to(gm.len.device))
    ab_dual = gm.algorithmic_bytes(aux_on=True)
    ab_prim = gm.algorithmic_bytes(aux_on=False)
    step_gbs = ab_dual["total"] / (ms_step / 1e3) / 1e9

    prim_ms = None
    if not args.no_primary_pass and dual:
        gm.len.copy_(len0)
        run(W, 0, aux_on=False)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(K, W, aux_on=False)
        e1.record(stream)
        torch.cuda.synchronize()
        prim_ms = e0.elapsed_time(e1) / K
        log(f"[bench] primary-only: {prim_ms:.3f} ms/step")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] calibration copy of 1 GiB done")
        del a, b

    read_ceiling = stream_read_ceiling(gm.k, attn_bytes_per_launch, attn_gbs, stream)

    cpu = None
    if not args.no_cpu_baseline:
        nl = args.cpu_layers or (2 if cfg.d >= 4096 else 4)
        log(f"[bench] CPU oracle baseline on a sample ({nl} layers)")
        del gm
        torch.cuda.empty_cache()
        cpu = cpu_baseline(cfg, nl)
        log(f"[bench] oracle: {cpu['value']:.4f} tok/s ({cpu['seconds_per_token']:.2f} s/token)")

    att_sha, lib_sha = source_hashes()
    measured = COUNTERS.get(cfg.name) if cfg.variant == 0 and not cfg.top_k_aux else None
    traffic = measured["attention_traffic_bytes_per_launch"] if (
        measured and att_sha == COUNTER_SOURCES["attention_source_sha256"]) else None
    counter_ratio = None
    if measured and lib_sha == COUNTER_SOURCES["library_sources_sha256"]:
        st = measured["step_traffic_bytes"]
        counter_ratio = st["dual"] / st["primary_only"]

    out = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded random-init weights, prefilled random K/V)",
        "config": {"workload": cfg.name, "layers": cfg.L, "d_model": cfg.d, "heads": cfg.H, "head_dim": cfg.Dh,
                   "ffn": cfg.F if not cfg.moe else None, "experts": cfg.E if cfg.moe else None,
                   "top_k": cfg.top_k if cfg.moe else None, "expert_ffn": cfg.Fe if cfg.moe else None,
                   "vocab": cfg.V, "global_batch": cfg.B, "context": cfg.ctx, "parallelism": "none (1 GPU)",
                   "variant": cfg.variant, "top_k_aux": cfg.top_k_aux if cfg.moe else None},
        "roofline": {"kernel": "attn_partial (shared-K/V dual-query attention, split-K pass)", "bound": "hbm",
                     "achieved": attn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": attn_gbs / PEAK_HBM_GBS,
                     "traffic": traffic, "avg_launch_ms": attn_avg_ms, "launches": attn_n,
                     "timed_every": TIMING_STRIDE, "algorithmic_bytes_per_launch": attn_bytes_per_launch},
        "step_bandwidth": {"algorithmic_bytes": ab_dual["total"], "achieved_GBs": step_gbs,
                           "frac": step_gbs / PEAK_HBM_GBS, "breakdown": ab_dual},
        "byte_ratio": {"analytic_dual_over_primary": ab_dual["total"] / ab_prim["total"], "counter": counter_ratio},
        "primary_only_ms_per_step": prim_ms,
        "dual_over_primary_time": (ms_step / prim_ms) if prim_ms else None,
        "device_status": status,
        "cpu_baseline": cpu,
    }
    out["read_ceiling"] = read_ceiling
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
