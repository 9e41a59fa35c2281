"""KDA benchmark on one MI355X.

One step = one kda_chunk_fwd call over the long-context prefill workload
B = 1, H = 32, T = 65536, d_k = d_v = 128, C = 64, bf16 q/k/v/beta, fp32
log-decay, S0 ~ N(0, 0.02^2), returning o and S_T (inputs already resident in
HBM).  The headline value is head-tokens per second (B*T*H / time).  The JSON
line also carries:
  * roofline: the call against HBM bandwidth (the pages' cost model puts the
    workload below the bf16 ridge point), its measured average launch time
    from HIP events on the launch stream, and the HBM traffic measured with
    rocprofv3 counters (stored under profiles/);
  * mfma: the pages' cost-model FLOPs as a fraction of the bf16 MFMA peak, and
    the counter-derived MFMA figures (executed bf16 MFMA operations, MFMA busy
    cycles) of the kernels, from rocprofv3 runs stored under profiles/;
  * prefill_c2: the B = 8, H = 16, T = 4096 prefill (S0 = 0) with its own
    roofline, MFMA figures and oracle timings (all host threads on the whole
    workload; one thread on a sample);
  * prefill_c1: the one-head fp32 T = 256 prefill, latency per call, and the
    one-thread oracle time of the same call;
  * decode: the recurrent decode step over 256 x 32 heads, state GB/s and %
    of HBM peak, plus four tokens per call through kda_recurrent_steps;
  * layer: the full token-mixing layer (d_model 2048, 16 heads, 32768
    tokens), its time, the KDA operator's share and the achieved TFLOP/s;
  * gate_variants: the B = 8 prefill with one decay per head and token (Gated
    DeltaNet) and with no decay (DeltaNet), through kda_chunk_fwd_gated;
  * full_attention_decode: the decode step of a NoPE MLA layer (MQA over a
    512-wide latent) at 1M tokens, and per sequence and layer against KDA's;
  * backward: kda_chunk_bwd on the B = 8 prefill workload (incoming gradients
    dL/do ~ N(0,1), dL/dS_T = 0), head-tokens/s, compulsory-HBM-bytes rate,
    and the gradient oracle timed on the host cores on the same workload;
  * cpu_baseline: the fp64 oracle timed on the host cores on the headline
    workload (thread count and host CPU model stated).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --workload c3|c2|c1|decode|layer|bwd|gdn|deltanet|mqa|dplr  (single-workload lines, for profiling)
       python bench.py --copy-calibration       (plain copy kernel for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz)
D, C = 128, 64
# Pages' cost model per head and token (page "Kimi K3论文：Kimi Linear", section 4):
# 6 T d^2 + 3 T C d + T C^2 FLOPs per head -> per head-token:
FLOP_PER_HEAD_TOKEN = 6 * D * D + 3 * C * D + C * C          # 126,976
# Compulsory HBM bytes per head-token for bf16 prefill: q, k, v (3 x 256),
# log-decay fp32 (512), beta bf16 (2), o bf16 (256).
BYTES_PER_HEAD_TOKEN_BF16 = 3 * 2 * D + 4 * D + 2 + 2 * D     # 1,538
BYTES_PER_HEAD_TOKEN_F32 = 3 * 4 * D + 4 * D + 4 + 4 * D      # 2,564
STATE_BYTES = 4 * D * D                                        # 65,536 per head
# Backward pass, compulsory HBM bytes per head-token (bf16): reads q, k, v, dO
# (4 x 256), log-decay fp32 (512), beta (2); writes dq, dk, dv (3 x 256),
# dlog-decay fp32 (512), dbeta (2).  Plus dS0 (fp32 state) per head.
BWD_BYTES_PER_HEAD_TOKEN = 4 * 2 * D + 4 * D + 2 + 3 * 2 * D + 4 * D + 2   # 2,820
# Decode: per head and step the state is read and written once, plus q, k, v
# (bf16), log-decay (fp32), beta (bf16) and o (bf16).
DECODE_BYTES_PER_HEAD = 2 * STATE_BYTES + 3 * 2 * D + 4 * D + 2 + 2 * D   # 132,610

PREFILL_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_32_amd", "csrc", "kda_prefill.hip")
DECODE_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_32_amd", "csrc", "kda_decode.hip")
BACKWARD_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_32_amd", "csrc", "kda_backward.hip")
DPLR_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_32_amd", "csrc", "kda_dplr.hip")
GEMM_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_32_amd", "csrc", "kda_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters.json")

WORKLOADS = {
    "c2": "c2_bf16_B8_H16_T4096",
    "c3": "c3_bf16_B1_H32_T65536",
    "c1": "c1_fp32_T256",
    "gdn": "c2_gdn_bf16_B8_H16_T4096",
    "deltanet": "c2_deltanet_bf16_B8_H16_T4096",
}
GATE_BYTES = {"channel": 4 * D, "head": 4, "none": 0}   # log-decay bytes per head-token


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_key, src_path):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    absent or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_sha256_16") != src_hash(src_path):
        return None
    return rec.get("bytes_per_launch")


def measured_counters(kernel_keys, src_path):
    """Counter-derived MFMA and LDS figures per launch (executed bf16 MFMA
    FLOPs = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16; MFMA busy fraction =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 256 CUs x 4 SIMDs),
    where rocprofv3 reports GRBM_GUI_ACTIVE summed over the 8 XCDs; LDS
    bank-conflict cycles per LDS instruction), summed over the kernels of one
    call, from committed rocprofv3 runs; None if absent or taken on other
    sources."""
    try:
        with open(COUNTER_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    parts = [recs.get(k) for k in kernel_keys]
    if any(p is None or p.get("src_sha256_16") != src_hash(src_path) for p in parts):
        return None
    us = sum(p["kernel_us"] for p in parts)
    flops = sum(p["mfma_bf16_flops"] for p in parts)
    busy = sum(p["mfma_busy_frac"] * p["kernel_us"] for p in parts) / us
    out = {"kernels": list(kernel_keys),
           "kernel_us": round(us, 2),
           "executed_mfma_bf16_flops": flops,
           "executed_mfma_tflops": round(flops / us / 1e6, 1),
           "executed_frac_of_bf16_peak": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4),
           "mfma_busy_frac": round(busy, 4),
           "source": sorted({p["source"] for p in parts})}
    if all("lds_bank_conflict_per_lds_inst" in p for p in parts):
        out["lds_bank_conflict_cycles_per_lds_inst"] = {k: p["lds_bank_conflict_per_lds_inst"]
                                                        for k, p in zip(kernel_keys, parts)}
    return out


def host_cpu():
    """Model name of the host CPU (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_launches(fn, steps, warmup):
    """Average time of fn() over `steps` back-to-back calls, from HIP events
    recorded on the current stream (the stream the kernels are launched on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3 / steps, wall


def prefill_line(name, steps, warmup, schedule="auto"):
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.PREFILL_CONFIGS[name]
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    log(f"[bench] generating inputs for {name}")
    inp = inputs.prefill_config(name)
    d = {n: (x.to("cuda:0") if x is not None else None) for n, x in inp.items()}
    o = torch.empty_like(d["v"])
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda:0")
    if schedule == "auto":
        nbytes = kda.workspace_size(B, T, H, kda.KDA_BF16 if cfg["dtype"] == "bfloat16" else kda.KDA_F32)
    else:
        nbytes = kda.scan_workspace_bytes(B, T, H) if schedule == "two_kernel" else 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0") if nbytes else None
    sched = "two_kernel" if ws is not None and cfg["dtype"] == "bfloat16" else "fused"
    if sched == "two_kernel" and nbytes > kda.scan_workspace_bytes(B, T, H):
        # the library's full workspace: segmented scan (16 heads or fewer) or,
        # for 24 to 48 heads (a multiple of 8), prep and scan in one launch
        sched = "pipelined" if B * H % 8 == 0 and 24 <= B * H <= 48 else "two_kernel_segmented"

    def step():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], out=o, S_T=S_T,
                      workspace=ws)

    log(f"[bench] timing {steps} steps after {warmup} warmup")
    t_kernel, wall = time_launches(step, steps, warmup)
    head_tokens = B * T * H
    per_ht = BYTES_PER_HEAD_TOKEN_BF16 if cfg["dtype"] == "bfloat16" else BYTES_PER_HEAD_TOKEN_F32
    gate = cfg.get("gate", "channel")
    per_ht += GATE_BYTES[gate] - GATE_BYTES["channel"]
    s0_bytes = STATE_BYTES * B * H if d["S0"] is not None else 0
    alg_bytes = head_tokens * per_ht + STATE_BYTES * B * H + s0_bytes
    flops = head_tokens * FLOP_PER_HEAD_TOKEN
    t_floor = max(alg_bytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    # kernels of one call: their rocprofv3 counter records under profiles/
    keys = ([f"chunk_fwd_{name}"] if sched in ("fused", "pipelined")
            else [f"chunk_fwd_{name}_prep", f"chunk_fwd_{name}_scan"])
    parts = [measured_traffic(key, PREFILL_KERNEL_SRC) for key in keys]
    traffic = sum(parts) if all(p is not None for p in parts) else None
    counters = measured_counters(keys, PREFILL_KERNEL_SRC)
    achieved = alg_bytes / t_kernel / 1e9
    return dict(
        inp=inp, t=t_kernel, wall=wall, head_tokens=head_tokens,
        value=head_tokens / t_kernel,
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": traffic,
                  "kernel": {"fused": "chunk_fwd_kernel (fused)",
                             "pipelined": "chunk_pipe_kernel (prep and scan roles in one launch)"}.get(
                                 sched, "chunk_fwd_kernel (prep) + chunk_scan_kernel"),
                  "alg_bytes_per_launch": alg_bytes,
                  "avg_launch_us": round(t_kernel * 1e6, 2)},
        mfma={"model_flops_per_launch": flops,
              "achieved_tflops": round(flops / t_kernel / 1e12, 2),
              "peak_tflops": BF16_PEAK_TFLOPS,
              "frac_of_bf16_peak": round(flops / t_kernel / 1e12 / BF16_PEAK_TFLOPS, 4),
              "frac_of_roofline": round(t_floor / t_kernel, 4),
              "counters": counters},
        config={"workload": f"kda_chunk_fwd {name}", "schedule": sched, "gate": gate,
                "B": B, "T": T, "H": H, "d_k": D, "d_v": D,
                "chunk": C, "dtype": cfg["dtype"], "S0": "N(0,%g)" % cfg["s0_std"] if d["S0"] is not None else "zero",
                "log_decay": ("none" if gate == "none" else
                              "-%g*softplus(N(0,1))" % cfg["g_scale"] + (" per head" if gate == "head" else ""))},
    )


def decode_line(steps, warmup):
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.DECODE_CONFIG
    N, H = cfg["N"], cfg["H"]
    nsteps = steps + warmup
    log(f"[bench] decode: {N}x{H} heads, {nsteps} steps of tokens")
    S = inputs.decode_state(N, H, s_std=cfg["s_std"], seed=cfg["seed"], device="cuda:0")
    toks = inputs.decode_tokens(N, H, nsteps, dtype=cfg["dtype"], seed=cfg["seed"], device="cuda:0")
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda:0")
    i = [0]

    def step():
        s = i[0] % nsteps
        kda.recurrent_step(toks["q"][s], toks["k"][s], toks["v"][s], toks["g"][s],
                           toks["beta"][s], S, out=o)
        i[0] += 1

    t, _ = time_launches(step, steps, warmup)
    alg = N * H * DECODE_BYTES_PER_HEAD
    gbs = alg / t / 1e9
    return {"workload": f"kda_recurrent_step {N}x{H} heads, fp32 128x128 state, bf16 tokens",
            "us_per_step": round(t * 1e6, 2), "state_gb_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "alg_bytes_per_step": alg,
            "traffic": measured_traffic("recurrent_step_decode", DECODE_KERNEL_SRC)}


def decode_latency_line(steps, warmup, N=1, H=32, per_graph=32):
    """Small-batch decode (N sequences x H heads): per-step time of eager calls
    through the Python binding against replays of a HIP graph holding
    `per_graph` captured steps (serving loops capture the step so that launch
    and binding overhead leave the per-token path)."""
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    S = inputs.decode_state(N, H, s_std=0.02, seed=4, device="cuda:0")
    toks = inputs.decode_tokens(N, H, 1, seed=4, device="cuda:0")
    tk = {n: toks[n][0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda:0")

    def step():
        kda.recurrent_step(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S, out=o)

    t_eager, _ = time_launches(step, steps * per_graph // 4, warmup)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            step()
    t_graph, _ = time_launches(graph.replay, max(steps // 4, 5), 2)
    return {"workload": f"kda_recurrent_step {N}x{H} heads (one decode step of a single sequence)",
            "eager_us_per_step": round(t_eager * 1e6, 2),
            "graph_us_per_step": round(t_graph / per_graph * 1e6, 2),
            "steps_per_graph": per_graph}


def multi_token_line(steps, warmup, m=4):
    """kda_recurrent_steps: m tokens per sequence in one call over 256 x 32
    heads (speculative or multi-token decoding; every token applied), against
    m single-token steps."""
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.DECODE_CONFIG
    N, H = cfg["N"], cfg["H"]
    S = inputs.decode_state(N, H, s_std=cfg["s_std"], seed=cfg["seed"], device="cuda:0")
    tk = inputs.decode_tokens(N, H, m, dtype=cfg["dtype"], seed=cfg["seed"], device="cuda:0")
    seq = {n: tk[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "beta")}   # [N, m, H, .]
    o = torch.empty((N, m, H, D), dtype=torch.bfloat16, device="cuda:0")
    t, _ = time_launches(lambda: kda.recurrent_steps(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"], S,
                                                     out=o), steps, warmup)
    alg = N * H * (2 * STATE_BYTES + m * (DECODE_BYTES_PER_HEAD - 2 * STATE_BYTES))
    return {"workload": f"kda_recurrent_steps {N}x{H} heads, m = {m} tokens per call (all applied)",
            "us_per_call": round(t * 1e6, 2), "us_per_token": round(t * 1e6 / m, 2),
            "alg_bytes_per_call": alg, "gb_s": round(alg / t / 1e9, 1),
            "frac_of_hbm_peak": round(alg / t / 1e9 / HBM_PEAK_GBS, 4)}


def mqa_line(steps, warmup, kda_decode=None):
    """Full-attention decode step at 1M context (MQA over a 512-wide bf16
    latent, the inference form of a NoPE MLA layer), and the comparison with
    KDA's decode step that the pages make at the model level."""
    import math
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.MQA_CONFIG
    B, T, H, Dc = cfg["B"], cfg["T"], cfg["H"], cfg["D"]
    log(f"[bench] mqa decode: B={B} T={T} H={H} D={Dc}")
    q, c = inputs.mqa_inputs(B, T, H, D=Dc, seed=cfg["seed"], device="cuda:0")
    o = torch.empty((B, H, Dc), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(int(kda.lib().kda_mqa_decode_workspace_size(B, T, H, Dc)), dtype=torch.uint8,
                     device="cuda:0")
    scale = 1.0 / math.sqrt(Dc)
    t, _ = time_launches(lambda: kda.mqa_decode(q, c, scale, out=o, workspace=ws), steps, warmup)
    alg = B * T * Dc * 2 + 2 * B * H * Dc * 2
    out = {"workload": f"kda_mqa_decode B={B} T={T} H={H} latent {Dc} bf16 (NoPE MLA as MQA)",
           "us_per_step": round(t * 1e6, 2), "alg_bytes_per_step": alg,
           "gb_s": round(alg / t / 1e9, 1), "frac_of_hbm_peak": round(alg / t / 1e9 / HBM_PEAK_GBS, 4)}
    if kda_decode is not None:
        # per sequence and layer: KDA's step amortised over the 256-sequence
        # batch, against this step for one sequence at 1M tokens
        t_kda = kda_decode["us_per_step"] / inputs.DECODE_CONFIG["N"]
        t_mla = out["us_per_step"] / B
        out["per_sequence_layer_us"] = {"kda": round(t_kda, 3), "full_attention_1m": round(t_mla, 2)}
        # a 3:1 hybrid group (3 KDA + 1 full-attention layer) against 4
        # full-attention layers: token-mixing time and cache per sequence
        out["hybrid_3to1_vs_full_attention"] = {
            "token_mixing_time_ratio": round(4 * t_mla / (t_mla + 3 * t_kda), 2),
            "cache_saving": round(1 - (T * Dc * 2 + 3 * 32 * STATE_BYTES) / (4 * T * Dc * 2), 4)}
    return out


# DPLR comparison path, compulsory HBM bytes per head-token (bf16): reads q,
# k, v, a, b (5 x 256), log-decay fp32 (512); writes o (256).
DPLR_BYTES_PER_HEAD_TOKEN = 5 * 2 * D + 4 * D + 2 * D          # 2,048


def dplr_line(steps, warmup, kda_ms=None):
    """The general diagonal-plus-low-rank recurrence at the B = 8, H = 16,
    T = 4096 shape (two kernels: prep + state scan), against KDA on the same
    shape: the comparison of the Kimi Linear page, section 4 (KDA about twice
    as fast as general DPLR)."""
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.DPLR_CONFIG
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    log(f"[bench] dplr: generating B={B} T={T} H={H}")
    inp = inputs.dplr_inputs(B, T, H, g_scale=cfg["g_scale"], s0_std=cfg["s0_std"], seed=cfg["seed"])
    d = {n: (x.to("cuda:0") if x is not None else None) for n, x in inp.items()}
    o = torch.empty_like(d["v"])
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(kda.dplr_workspace_size(B, T, H), dtype=torch.uint8, device="cuda:0")
    t, _ = time_launches(lambda: kda.dplr_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["g"], None,
                                                    out=o, S_T=S_T, workspace=ws), steps, warmup)
    ht = B * T * H
    alg = ht * DPLR_BYTES_PER_HEAD_TOKEN + STATE_BYTES * B * H
    parts = [measured_traffic(key, src) for key, src in
             (("dplr_prep", DPLR_KERNEL_SRC), ("dplr_scan", PREFILL_KERNEL_SRC))]
    traffic = sum(parts) if all(p is not None for p in parts) else None
    out = {"workload": f"kda_dplr_chunk_fwd B={B} T={T} H={H} bf16 (a = beta ka, b = alpha kb, ka, kb free)",
           "ms_per_step": round(t * 1e3, 4), "head_tokens_per_s": round(ht / t, 1),
           "alg_bytes_per_step": alg, "frac_of_hbm_peak": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
           "traffic_bytes_per_step": traffic,
           "traffic_gb_s": None if traffic is None else round(traffic / t / 1e9, 1),
           "workspace_bytes": ws.numel()}
    kda2 = prefill_line(WORKLOADS["c2"], steps, warmup, "two_kernel")
    out["kda_same_shape_ms"] = {"two_kernel": round(kda2["t"] * 1e3, 4)}
    if kda_ms is not None:
        out["kda_same_shape_ms"]["library_schedule"] = round(kda_ms, 4)
    best = min(out["kda_same_shape_ms"].values())
    out["dplr_over_kda"] = {k: round(t * 1e3 / v, 2) for k, v in out["kda_same_shape_ms"].items()}
    out["dplr_over_kda_best"] = round(t * 1e3 / best, 2)
    return out


def layer_line(steps, warmup):
    """The full token-mixing layer (projections, conv/activations, gates, KDA,
    gated RMSNorm, output projection) on the 32768-token, d_model 2048, 16-head
    workload; also times the KDA operator alone on the layer's own inputs."""
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    cfg = inputs.LAYER_CONFIG
    B, T, dm, H = cfg["B"], cfg["T"], cfg["d_model"], cfg["H"]
    rank = D
    log(f"[bench] layer: generating B={B} T={T} d_model={dm} H={H}")
    inp = inputs.layer_inputs(B=B, T=T, d_model=dm, H=H, seed=cfg["seed"], gate_rank=rank)
    dev = torch.device("cuda", 0)
    x = inp["x"].to(dev)
    W = {n: inp[n].to(dev) for n in kda.LAYER_WEIGHTS}
    total, _ = kda.layer_workspace_layout(B, T, dm, H, rank)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=dev)
    _, iv = kda.layer_fwd(x, W, H, out=y, workspace=ws, intermediates=True)
    t_layer, _ = time_launches(lambda: kda.layer_fwd(x, W, H, out=y, workspace=ws), steps, warmup)
    o = torch.empty_like(iv["v"])
    t_kda, _ = time_launches(lambda: kda.chunk_fwd(iv["q"], iv["k"], iv["v"], iv["g"], iv["beta"],
                                                   None, out=o, return_state=False), steps, warmup)
    hd = H * D
    gemm_flops = 2 * B * T * (dm * (4 * hd + rank + H) + rank * hd + hd * dm)
    kda_flops = B * T * H * FLOP_PER_HEAD_TOKEN
    return {"workload": f"kda_layer_fwd B={B} T={T} d_model={dm} H={H}x{D} gate rank {rank}, bf16",
            "ms_per_layer": round(t_layer * 1e3, 4),
            "tokens_per_s": round(B * T / t_layer, 1),
            "kda_operator_ms": round(t_kda * 1e3, 4),
            "rest_ms": round((t_layer - t_kda) * 1e3, 4),
            "model_flops": gemm_flops + kda_flops,
            "achieved_tflops": round((gemm_flops + kda_flops) / t_layer / 1e12, 1),
            "frac_of_bf16_peak": round((gemm_flops + kda_flops) / t_layer / 1e12 / BF16_PEAK_TFLOPS, 4),
            "projection_gemm_counters": measured_counters(["kda_layer_gemm_qkvg", "kda_layer_gemm_o"],
                                                          GEMM_KERNEL_SRC)}


def backward_line(steps, warmup, with_cpu=False, wl="c2"):
    """kda_chunk_bwd on the B = 8, H = 16, T = 4096 prefill workload (or, with
    wl = "gdn" / "deltanet", the same shape with the other two gates)."""
    import torch
    import gated_delta_rule_32_amd as kda
    from gated_delta_rule_32_amd import inputs

    name = WORKLOADS[wl]
    cfg = inputs.PREFILL_CONFIGS[name]
    gate = cfg.get("gate", "channel")
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    log(f"[bench] backward: generating inputs for {name}")
    inp = inputs.prefill_config(name)
    gr = inputs.grad_inputs(B, T, H, seed=cfg["seed"])
    d = {n: (x.to("cuda:0") if x is not None else None) for n, x in {**inp, **gr}.items()}
    ws = torch.empty(kda.bwd_workspace_size(B, T, H), dtype=torch.uint8, device="cuda:0")

    def step():
        kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], d["dO"], d["dS_T"],
                      workspace=ws)

    log(f"[bench] backward: timing {steps} steps after {warmup} warmup")
    t, _ = time_launches(step, steps, warmup)
    ht = B * T * H
    # the log-decay is read once and its gradient written once
    alg = ht * (BWD_BYTES_PER_HEAD_TOKEN + 2 * (GATE_BYTES[gate] - GATE_BYTES["channel"])) + STATE_BYTES * B * H
    gbs = alg / t / 1e9
    if wl != "c2":
        return {"workload": f"kda_chunk_bwd {name} (dL/do ~ N(0,1), dL/dS_T = 0)", "gate": gate,
                "ms_per_step": round(t * 1e3, 4), "head_tokens_per_s": round(ht / t, 1),
                "alg_bytes_per_step": alg, "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    # measured HBM traffic of the four kernels (rocprofv3 counters, committed
    # under profiles/), when taken on the current sources
    parts = [measured_traffic(key, src) for key, src in
             (("chunk_bwd_prep", PREFILL_KERNEL_SRC), ("chunk_bwd_fwd_scan", PREFILL_KERNEL_SRC),
              ("chunk_bwd_scan", BACKWARD_KERNEL_SRC), ("chunk_bwd_grad", BACKWARD_KERNEL_SRC))]
    traffic = sum(parts) if all(p is not None for p in parts) else None
    out = {"workload": f"kda_chunk_bwd {name} (dL/do ~ N(0,1), dL/dS_T = 0)",
           "ms_per_step": round(t * 1e3, 4), "head_tokens_per_s": round(ht / t, 1),
           "alg_bytes_per_step": alg, "compulsory_gb_s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "traffic_bytes_per_step": traffic,
           "traffic_gb_s": None if traffic is None else round(traffic / t / 1e9, 1),
           "workspace_bytes": ws.numel()}
    if with_cpu:
        from oracle import kda_ref
        threads = kda_ref.max_threads()
        args = [kda_ref._f64(inp[n]) for n in ("q", "k", "v", "g", "beta")]
        log(f"[bench] backward cpu baseline: gradient oracle, {threads} threads")
        t0 = time.perf_counter()
        kda_ref.recurrent_grad(*args, None, kda_ref._f64(gr["dO"]), None, nthreads=threads)
        dt = time.perf_counter() - t0
        out["cpu_oracle"] = {"value": round(ht / dt, 1), "unit": "head-tokens/s", "cores": threads,
                             "kind": "oracle", "cpu_model": host_cpu(),
                             "sample": f"whole workload: {B}x{H} heads x {T} tokens, fp64 reverse-mode "
                                       f"recurrence (C, -O2, OpenMP over heads), {dt:.2f} s wall"}
    return out


def _oracle_threads():
    """Threads the numpy / BLAS parts of the oracle may use on this host."""
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def _oracle_timing(fn, units, unit, cores, sample):
    """The oracle as it stands, timed on the host over one bounded sample."""
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": round(units / dt, 1), "unit": unit, "cores": cores, "kind": "oracle",
            "cpu_model": host_cpu(), "sample": f"{sample}, {dt:.2f} s wall"}


def oracle_timings():
    """The oracles of the other measured paths, each on a sample of about a
    second of CPU work (inputs drawn as for the GPU lines)."""
    import numpy as np
    import torch
    from gated_delta_rule_32_amd import inputs
    from oracle import dplr_ref, kda_layer_ref, kda_ref, mqa_ref
    out = {}
    threads = kda_ref.max_threads()
    # decode: 32 sequences x 32 heads, 64 steps, through the recurrence from the decode state
    N, H, steps = 32, 32, 64
    S0 = inputs.decode_state(N, H, s_std=0.02, seed=4)
    tk = inputs.decode_tokens(N, H, steps, seed=4)
    args = [kda_ref._f64(tk[n]).transpose(1, 0, 2, 3) for n in ("q", "k", "v", "g")]
    beta = kda_ref._f64(tk["beta"]).transpose(1, 0, 2)
    s0 = kda_ref._f64(S0)
    log(f"[bench] oracle timing: decode {N}x{H} heads x {steps} steps")
    out["decode"] = _oracle_timing(lambda: kda_ref.recurrent(*args[:3], args[3], beta, s0, nthreads=threads),
                                   N * H * steps * DECODE_BYTES_PER_HEAD / 1e9, "GB/s (state bytes)", threads,
                                   f"{N}x{H} heads x {steps} steps of the fp64 recurrence (C, OpenMP)")
    # gate variants: 4 x 16 heads x 4096 tokens each
    for wl, gate in (("gdn", "head"), ("deltanet", "none")):
        inp = inputs.prefill_inputs(4, 4096, 16, g_scale=0.05, seed=2, gate=gate)
        g = (np.zeros(inp["q"].shape) if inp["g"] is None else
             np.repeat(kda_ref._f64(inp["g"])[..., None], D, axis=-1))
        a = [kda_ref._f64(inp[n]) for n in ("q", "k", "v")] + [g, kda_ref._f64(inp["beta"])]
        log(f"[bench] oracle timing: {wl}")
        out[wl] = _oracle_timing(lambda: kda_ref.recurrent(*a, None, nthreads=threads), 64 * 4096,
                                 "head-tokens/s", threads, "4x16 heads x 4096 tokens of the fp64 recurrence "
                                 "(decay copied to every channel or zero)")
    # DPLR: 2 heads x 4096 tokens, numpy
    dp = inputs.dplr_inputs(1, 4096, 2, seed=7)
    log("[bench] oracle timing: dplr")
    out["dplr"] = _oracle_timing(lambda: dplr_ref.recurrent(*(dp[n] for n in ("q", "k", "v", "a", "b", "g")), None),
                                 2 * 4096, "head-tokens/s", 1, "2 heads x 4096 tokens of the fp64 DPLR "
                                 "recurrence (numpy, one token at a time)")
    # full-attention decode: 32 heads over 2^18 cached tokens
    Tm = 1 << 18
    q, c = inputs.mqa_inputs(1, Tm, 32, seed=6)
    log("[bench] oracle timing: full-attention decode")
    out["full_attention_decode"] = _oracle_timing(lambda: mqa_ref.decode(q, c, 1.0 / 512 ** 0.5), Tm * 1024 / 1e9,
                                                  "GB/s (cache bytes)", _oracle_threads(),
                                                  f"1 sequence, 32 heads over {Tm} cached tokens (fp64 numpy / BLAS)")
    # layer: 1024 tokens with the full-size weights
    Tl = 1024
    li = inputs.layer_inputs(B=1, T=Tl, d_model=2048, H=16, seed=5, gate_rank=D)
    W = {n: li[n] for n in li if n != "x"}
    log("[bench] oracle timing: layer")
    out["layer"] = _oracle_timing(lambda: kda_layer_ref.layer_forward(li["x"], W, 16), Tl, "tokens/s",
                                  _oracle_threads(), f"{Tl} tokens, d_model 2048, 16 heads, full-size weights "
                                  "(fp64 numpy / BLAS and the C recurrence)")
    del torch
    return out


def cpu_baseline(inp, threads=None, batches=None, label="whole workload"):
    """The fp64 oracle as it stands, on the host cores (``threads``: all of
    them by default), over the workload's batches ``batches`` (all by
    default): head-tokens per second."""
    from oracle import kda_ref
    if batches is not None:
        inp = {n: (None if x is None else x[batches]) for n, x in inp.items()}
    B, T, H, _ = inp["q"].shape
    arrs = [kda_ref._f64(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    S0 = kda_ref._f64(inp["S0"])
    threads = threads or kda_ref.max_threads()
    reps = max(1, int(2e5 // (B * T * H)))      # tiny workloads: repeat to reach ~a second
    log(f"[bench] cpu oracle: {B}x{H} heads x {T} tokens, {threads} threads, {reps} rep(s)")
    t0 = time.perf_counter()
    for _ in range(reps):
        kda_ref.recurrent(*arrs, S0, nthreads=threads)
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(B * T * H / dt, 1), "unit": "head-tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": host_cpu(),
            "sample": f"{label}: {B}x{H} heads x {T} tokens, fp64 sequential recurrence "
                      f"(C, -O2, OpenMP over heads), {dt:.3f} s wall per call"
                      + (f" (mean of {reps} calls)" if reps > 1 else "")}


def c2_entry(args):
    """The B = 8, H = 16, T = 4096 prefill (S0 = 0) with its own roofline,
    counters and oracle timings."""
    pre = prefill_line(WORKLOADS["c2"], args.steps, args.warmup, args.schedule)
    out = {"workload": pre["config"]["workload"], "config": pre["config"],
           "ms_per_step": round(pre["t"] * 1e3, 4), "head_tokens_per_s": round(pre["value"], 1),
           "roofline": pre["roofline"], "mfma": pre["mfma"]}
    if not args.no_cpu:
        out["cpu_oracle"] = cpu_baseline(pre["inp"])
        # one thread on one of the 8 batches (16 heads x 4096 tokens)
        out["cpu_oracle_1thread"] = cpu_baseline(pre["inp"], threads=1, batches=slice(0, 1),
                                                 label="batch 0 of 8 (1/8 of the workload)")
    return out, pre


def c1_entry(args):
    """The one-head fp32 T = 256 prefill: latency of one call (a parity
    workload; it occupies one workgroup of the GPU)."""
    pre = prefill_line(WORKLOADS["c1"], max(args.steps, 200), args.warmup)
    out = {"workload": pre["config"]["workload"], "config": pre["config"],
           "us_per_call": round(pre["t"] * 1e6, 2), "head_tokens_per_s": round(pre["value"], 1)}
    if not args.no_cpu:
        out["cpu_oracle_1thread"] = cpu_baseline(pre["inp"], threads=1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-gates", action="store_true")
    ap.add_argument("--no-mqa", action="store_true")
    ap.add_argument("--no-dplr", action="store_true")
    ap.add_argument("--workload", choices=["c3", "c2", "c1", "decode", "layer", "bwd", "gdn", "deltanet", "mqa", "dplr"],
                    default=None,
                    help="time one workload only (profiling runs)")
    ap.add_argument("--schedule", choices=["auto", "fused", "two_kernel"], default="auto",
                    help="prefill schedule (auto: the library's preferred one)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for HBM counter scaling) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the KDA heads shard across GPUs with no communication, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()

    if args.copy_calibration:
        n = 1 << 28   # 256 Mi floats = 1 GiB
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return

    if args.workload == "decode":
        dec = decode_line(args.steps, args.warmup)
        print(json.dumps({"metric": "KDA decode state GB/s", **dec}))
        return

    if args.workload == "bwd":
        bwd = backward_line(args.steps, args.warmup)
        print(json.dumps({"metric": "KDA backward head-tokens/s", **bwd}))
        return

    if args.workload == "dplr":
        print(json.dumps({"metric": "DPLR chunked forward", **dplr_line(args.steps, args.warmup)}))
        return

    if args.workload == "mqa":
        print(json.dumps({"metric": "full-attention decode step", **mqa_line(args.steps, args.warmup)}))
        return

    if args.workload == "layer":
        lay = layer_line(args.steps, args.warmup)
        print(json.dumps({"metric": "KDA layer tokens/s", **lay}))
        return

    name = WORKLOADS[args.workload or "c3"]
    pre = prefill_line(name, args.steps, args.warmup, args.schedule)
    line = {
        "metric": "KDA prefill tokens/s/head-layer (% MFMA peak); decode state GB/s (% HBM)",
        "value": round(pre["value"], 1),
        "unit": "head-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(pre["t"] * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if pre["config"]["dtype"] == "bfloat16" else "f32",
        "data": "synthetic",
        "config": pre["config"],
        "roofline": pre["roofline"],
        "mfma": pre["mfma"],
    }
    c2 = None
    if args.workload is None:
        line["prefill_c2"], c2 = c2_entry(args)
        line["prefill_c1"] = c1_entry(args)
    if args.workload is None and not args.no_decode:
        line["decode"] = decode_line(max(args.steps, 20), args.warmup)
        line["decode"]["small_batch"] = decode_latency_line(max(args.steps, 20), args.warmup)
        line["decode"]["multi_token"] = multi_token_line(max(args.steps, 20), args.warmup)
    if args.workload is None and not args.no_mqa:
        line["full_attention_decode"] = mqa_line(max(args.steps, 20), args.warmup, line.get("decode"))
    if args.workload is None and not args.no_layer:
        line["layer"] = layer_line(min(args.steps, 20), args.warmup)
    if args.workload is None and not args.no_gates:
        line["gate_variants"] = {}
        for wl in ("gdn", "deltanet"):
            r = prefill_line(WORKLOADS[wl], args.steps, args.warmup)
            line["gate_variants"][wl] = {"workload": r["config"]["workload"], "gate": r["config"]["gate"],
                                         "ms_per_step": round(r["t"] * 1e3, 4),
                                         "head_tokens_per_s": round(r["value"], 1),
                                         "alg_bytes_per_launch": r["roofline"]["alg_bytes_per_launch"],
                                         "hbm_frac": r["roofline"]["frac"],
                                         "mfma_frac": r["mfma"]["frac_of_bf16_peak"]}
            if not args.no_bwd:
                line["gate_variants"][wl]["backward"] = backward_line(min(args.steps, 20), args.warmup, wl=wl)
    if args.workload is None and not args.no_dplr:
        line["dplr_comparison"] = dplr_line(args.steps, args.warmup, c2["t"] * 1e3)
    if args.workload is None and not args.no_bwd:
        line["backward"] = backward_line(min(args.steps, 20), args.warmup, with_cpu=not args.no_cpu)
    if not args.no_cpu and args.workload is None:
        line["cpu_baseline"] = cpu_baseline(pre["inp"])
        del pre["inp"]
        orc = oracle_timings()
        for key, target in (("decode", line.get("decode")), ("full_attention_decode", line.get("full_attention_decode")),
                            ("layer", line.get("layer")), ("dplr", line.get("dplr_comparison"))):
            if target is not None:
                target["cpu_oracle"] = orc[key]
        for wl in ("gdn", "deltanet"):
            if wl in line.get("gate_variants", {}):
                line["gate_variants"][wl]["cpu_oracle"] = orc[wl]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
