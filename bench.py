"""Benchmark: QLoRA gated-MLP (or q/k/v) forward + backward on one MI355X.

Workload (default): Llama-7B MLP block, 8192 tokens (4 x 2048) x 4096 ->
11008 -> 4096, NF4 (blocksize 64) gate/up/down, LoRA rank 16, s = 1, SwiGLU,
synthetic seeded inputs already resident in HBM. One step = qlora_mlp_fwd +
qlora_mlp_bwd (every kernel of the path). The metric counts algorithmic
FLOPs only: six base products 2*m*d*h plus the LoRA products (recompute,
dequant and elementwise work are not counted).

Other workloads: the Mistral-7B / Gemma-7B MLP shapes, and the q/k/v
projections of one input at the Mistral-7B (4096 -> 4096 / 1024 / 1024) and
Llama-7B (3 x 4096) shapes, 8192 tokens; one step = qlora_qkv_fwd +
qlora_qkv_bwd, FLOPs 4*m*d*n + 6*m*r*(d + n) per projection.

Prints ONE JSON line. Extra fields: roofline (the base-GEMM kernel, timed
live with HIP events on its launch stream) and cpu_baseline (the fp64 CPU
oracle on a bounded token sample of the same workload).

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama7b_mlp]
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (no sparsity)
METRIC = "QLoRA MLP fwd+bwd TFLOP/s + % bf16 MFMA peak, Llama-7B shape, 8192 tok"
METRIC_QKV = "QLoRA q/k/v fwd+bwd TFLOP/s + % bf16 MFMA peak, {model} shape, 8192 tok"
MLP_WORKLOADS = ["llama7b_mlp", "mistral7b_mlp", "gemma7b_mlp"]
QKV_WORKLOADS = ["mistral7b_qkv", "llama7b_qkv"]
LINEAR_WORKLOADS = ["llama7b_q_proj", "mistral7b_kv_proj"]
QUANT_WORKLOAD = "llama7b_mlp_quantize"
FAST_WORKLOADS = ["llama7b_norm_rope_xent", "gemma7b_norm_rope_xent"]
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
QUANT_BYTES_PER_WEIGHT = 2 + 0.5 + 4 / 64   # bf16 in; codes + fp32 absmax out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama7b_mlp",
                   choices=MLP_WORKLOADS + QKV_WORKLOADS + LINEAR_WORKLOADS + [QUANT_WORKLOAD]
                   + FAST_WORKLOADS)
    p.add_argument("--tokens", type=int, default=0,
                   help="token count instead of the workload's 8192 (e.g. one GPU's data-parallel share)")
    p.add_argument("--rank", type=int, default=0,
                   help="LoRA rank r instead of the workload's 16 (1..64)")
    p.add_argument("--mode", default="auto", choices=["auto", "fused", "staged"])
    p.add_argument("--base", default="nf4", choices=["nf4", "bf16"],
                   help="base weights: NF4 (QLoRA, default) or bf16 (16-bit LoRA variant)")
    p.add_argument("--cpu-tokens", type=int, default=2048,
                   help="token sample of the CPU oracle baseline (0 = skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 3 times (counter calibration)")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch.

    Profiled with the same rocprofv3 counters as the benchmark, it gives the
    factor between what FETCH_SIZE / WRITE_SIZE report and true HBM bytes.
    """
    import torch
    n = 1 << 29                      # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": 2 * n, "launches": 3}))


def mlp_flops(m, d, h, r):
    """Algorithmic FLOPs of one MLP fwd+bwd: six base products 2*m*d*h (no base
    weight gradient) plus 2*m*r*(in+out) per LoRA projection forward and twice
    that backward."""
    return 6 * 2 * m * d * h + 3 * 3 * 2 * m * r * (d + h)


def linear_flops(m, k, n, r):
    """Algorithmic FLOPs of one linear layer forward + backward: two base products
    2*m*k*n, 2*m*r*(k+n) of LoRA forward and twice that backward."""
    return 4 * m * k * n + 6 * m * r * (k + n)


def qkv_flops(m, d, ns, r):
    """Algorithmic FLOPs of the q/k/v forward + backward: per projection two
    base products 2*m*d*n and 2*m*r*(d+n) of LoRA forward, twice that backward."""
    return sum(4 * m * d * n + 6 * m * r * (d + n) for n in ns)


def code_digest(path):
    """SHA-256 of a C++ source with comments and whitespace removed, so that a
    comment edit does not count as a kernel change."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def gemm_traffic(lib_src_dir, workload, mode):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when it was taken on another workload or dequant mode, or the
    kernel code changed since."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    h = code_digest(os.path.join(lib_src_dir, "gemm.hip"))
    for rec in json.load(open(path)):
        if (rec.get("gemm_hip_code_sha256") == h and rec.get("workload_name") == workload
                and rec.get("dequant_mode") == mode):
            return rec.get("hbm_bytes_per_launch")
    return None


def host_cpu():
    """(model name, logical CPUs the process may run on) of the host."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(cfg, d, tokens):
    """fp64 oracle (as it stands) on the first `tokens` tokens of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import nf4 as onf4
    from oracle import qlora as oq

    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    t0 = time.perf_counter()
    W = {wn: onf4.dequant_f64(d[wn + "_codes"].numpy(), d[wn + "_absmax"].numpy())
         for wn in ("Wg", "Wu", "Wd")}
    t_dq = time.perf_counter() - t0
    L = [f64(d[k]) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")]
    X, dY = f64(d["X"][:tokens]), f64(d["dY"][:tokens])
    args = (W["Wg"], W["Wu"], W["Wd"], *L, cfg.s, cfg.act)
    t0 = time.perf_counter()
    _, sv = oq.mlp_fwd(X, *args)
    oq.mlp_bwd(dY, X, sv, *args)
    t = time.perf_counter() - t0 + t_dq     # a step dequantizes its weights too
    flops = oq.mlp_algorithmic_flops(tokens, cfg.d, cfg.h, cfg.r)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model, nproc = host_cpu()
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "nproc": nproc,
            "sample": f"{tokens} of {cfg.m} tokens with the full {cfg.name} weights, fp64 numpy: "
                      f"weight dequant {t_dq:.2f} s + fwd/bwd {t - t_dq:.2f} s",
            "tokens_per_s": round(tokens / t, 3), "seconds": round(t, 3)}


def cpu_baseline_qkv(cfg, d, tokens):
    """fp64 oracle (as it stands) on the first `tokens` tokens of the q/k/v workload."""
    import torch
    from threadpoolctl import threadpool_info

    from oracle import nf4 as onf4
    from oracle import qlora as oq

    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    t0 = time.perf_counter()
    Ws = [onf4.dequant_f64(d["W" + p + "_codes"].numpy(), d["W" + p + "_absmax"].numpy())
          for p in "qkv"]
    t_dq = time.perf_counter() - t0
    As = [f64(d["A" + p]) for p in "qkv"]
    Bs = [f64(d["B" + p]) for p in "qkv"]
    X = f64(d["X"][:tokens])
    dYs = [f64(d["dY" + p][:tokens]) for p in "qkv"]
    t0 = time.perf_counter()
    _, Us = oq.qkv_fwd(X, Ws, As, Bs, cfg.s)
    oq.qkv_bwd(dYs, X, Us, Ws, As, Bs, cfg.s)
    t = time.perf_counter() - t0 + t_dq
    flops = oq.qkv_algorithmic_flops(tokens, cfg.d, (cfg.n_q, cfg.n_k, cfg.n_v), cfg.r)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model, nproc = host_cpu()
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "nproc": nproc,
            "sample": f"{tokens} of {cfg.m} tokens with the full {cfg.name} weights, fp64 numpy: "
                      f"weight dequant {t_dq:.2f} s + fwd/bwd {t - t_dq:.2f} s",
            "tokens_per_s": round(tokens / t, 3), "seconds": round(t, 3)}


def bench_quantize(a):
    """NF4 quantization of the three Llama-7B MLP weights (gate, up [11008][4096],
    down [4096][11008]) from bf16, one step = the three qlora_nf4_quantize calls.
    HBM-bound: 2 B read and 0.5 + 4/64 B written per weight."""
    import torch

    import qlora_fine_tuning_amd as Q
    from qlora_fine_tuning_amd import inputs as I

    dev = "cuda:0"
    cfg = I.LLAMA_MLP
    shapes = {"Wg": (cfg.h, cfg.d), "Wu": (cfg.h, cfg.d), "Wd": (cfg.d, cfg.h)}
    Ws = {wn: I.normal_bf16(wn, sh, 0.02) for wn, sh in shapes.items()}
    Wd = {wn: w.to(dev) for wn, w in Ws.items()}
    outs = {wn: Q.nf4_quantize(w) for wn, w in Wd.items()}

    def step():
        for wn, w in Wd.items():
            Q.nf4_quantize(w, out=outs[wn])

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / a.steps
    nw = sum(n * k for n, k in shapes.values())
    gbs = nw * QUANT_BYTES_PER_WEIGHT / (ms / 1e3) / 1e9
    out = {
        "metric": "NF4 quantize (bf16 -> codes + fp32 absmax) GB/s, Llama-7B MLP weights",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->nf4", "data": "synthetic",
        "config": {"workload": QUANT_WORKLOAD, "weights": [list(v) for v in shapes.values()],
                   "blocksize": 64, "global_batch": None, "parallelism": "none (1 GPU)"},
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "hbm", "kernel": "nf4_quantize_kernel", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_weight": QUANT_BYTES_PER_WEIGHT,
                     "launches_per_step": 3, "avg_launch_ms": round(ms / 3, 4)},
    }
    if a.cpu_tokens > 0:   # oracle quantizer on a bounded sample of gate rows
        from oracle import nf4 as onf4
        rows = 4096
        bits = Ws["Wg"][:rows].contiguous().view(torch.int16).numpy().view("uint16")
        t0 = time.perf_counter()
        onf4.quantize(bits)
        t = time.perf_counter() - t0
        model, nproc = host_cpu()
        out["cpu_baseline"] = {"value": round(rows * cfg.d * QUANT_BYTES_PER_WEIGHT / t / 1e9, 4),
                               "unit": "GB/s", "cores": 1, "kind": "oracle", "cpu_model": model,
                               "nproc": nproc,
                               "sample": f"{rows} of {cfg.h} gate rows ({rows * cfg.d} weights), fp64 numpy",
                               "seconds": round(t, 3)}
    print(json.dumps(out), flush=True)


def bench_fast(a):
    """RMS layernorm, RoPE (q and k) and cross entropy, forward + backward, at one
    model's sizes and 8192 tokens (4 x 2048). HBM-bound: value = algorithmic
    bytes (every operand read once, every output written once) / step time."""
    import numpy as np
    import torch

    import qlora_fine_tuning_amd as Q
    from qlora_fine_tuning_amd import inputs as I

    dev = "cuda:0"
    llama = a.workload == "llama7b_norm_rope_xent"
    m = 8192
    d, hq, hk, hd, V, eps, gemma = ((4096, 32, 32, 128, 32000, 1e-6, False) if llama
                                    else (3072, 16, 16, 256, 256000, 1e-6, True))
    X = I.normal_bf16("X", (m, d), 1.0).to(dev)
    w = (I.normal_bf16("W", (d,), 0.1) + (0 if gemma else 1)).to(torch.bfloat16).to(dev)
    dY = I.normal_bf16("dY", (m, d), 1.0).to(dev)
    q = I.normal_bf16("Wk", (m, hq, hd), 1.0).to(dev)
    k = I.normal_bf16("Wv", (m, hk, hd), 1.0).to(dev)
    pos = (torch.arange(m, dtype=torch.int64) % 2048).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(I.SEED)   # seeded device draw: the Gemma logits are 2.1e9 values
    logits = (torch.randn((m, V), generator=gen, device=dev) * 2.0).to(torch.bfloat16)
    g = np.random.default_rng(I.SEED)
    lab_np = g.integers(0, V, size=m).astype(np.int64)
    lab_np[::2048] = -100                                   # no target after each sequence's last token
    labels = torch.from_numpy(lab_np).to(dev)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    e = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    parts = ["rmsnorm_fwd", "rmsnorm_bwd", "rope_fwd", "rope_bwd", "xent_fwd", "xent_bwd"]
    nq, nk = m * hq * hd, m * hk * hd
    alg = {"rmsnorm_fwd": 4 * m * d + 4 * m + 2 * d, "rmsnorm_bwd": 6 * m * d + 4 * m + 2 * d,
           "rope_fwd": 4 * (nq + nk) + 8 * m, "rope_bwd": 4 * (nq + nk) + 8 * m,
           "xent_fwd": 2 * m * V + 16 * m, "xent_bwd": 4 * m * V + 16 * m}

    def step(evs=None):
        def mark(i):
            if evs is not None:
                evs[i].record()
        mark(0)
        Y, rstd = Q.rmsnorm_fwd(X, w, eps, gemma)
        mark(1)
        Q.rmsnorm_bwd(dY, X, rstd, w, gemma)
        mark(2)
        Q.rope_fwd(q, pos, out=qo)
        Q.rope_fwd(k, pos, out=ko)
        mark(3)
        Q.rope_bwd(qo, pos, out=qo, inplace=True)
        Q.rope_bwd(ko, pos, out=ko, inplace=True)
        mark(4)
        f = Q.cross_entropy_fwd(logits, labels)
        mark(5)
        Q.cross_entropy_bwd(logits, labels, f)
        mark(6)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = e(), e()
    ev0.record()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / a.steps
    per = {p_: 0.0 for p_ in parts}
    for _ in range(3):   # per-kernel breakdown, separate from the timed steps
        evs = [e() for _ in range(7)]
        step(evs)
        torch.cuda.synchronize()
        for i, p_ in enumerate(parts):
            per[p_] += evs[i].elapsed_time(evs[i + 1]) / 3
    # the fused cross-entropy forward + backward, timed on its own
    xf = [e(), e()]
    for _ in range(2):
        Q.cross_entropy_fused(logits, labels)
    xf[0].record()
    for _ in range(5):
        Q.cross_entropy_fused(logits, labels)
    xf[1].record()
    torch.cuda.synchronize()
    fused_ms = xf[0].elapsed_time(xf[1]) / 5
    fused_alg = 4 * m * V + 16 * m
    total = sum(alg.values())
    gbs = total / (ms / 1e3) / 1e9
    dom = "xent_bwd"
    dom_gbs = alg[dom] / (per[dom] / 1e3) / 1e9
    out = {
        "metric": f"RMS layernorm + RoPE + cross entropy fwd+bwd GB/s, {'Llama' if llama else 'Gemma'}-7B sizes, 8192 tok",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp32 arithmetic)", "data": "synthetic",
        "config": {"workload": a.workload, "tokens": m, "d": d, "q_heads": hq, "k_heads": hk,
                   "head_dim": hd, "vocab": V, "norm": "1+w" if gemma else "w", "global_batch": m,
                   "parallelism": "none (1 GPU)"},
        "wall_s_timed": round(wall, 3),
        "kernels": {p_: {"us": round(per[p_] * 1e3, 1),
                         "GB/s": round(alg[p_] / (per[p_] / 1e3) / 1e9, 1)} for p_ in parts},
        "xent_fused": {"us": round(fused_ms * 1e3, 1),
                       "GB/s": round(fused_alg / (fused_ms / 1e3) / 1e9, 1),
                       "vs_fwd_plus_bwd": round((per["xent_fwd"] + per["xent_bwd"]) / fused_ms, 3)},
        "roofline": {"bound": "hbm", "kernel": "xent_bwd_kernel", "achieved": round(dom_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "algorithmic_bytes": alg[dom],
                     "avg_launch_ms": round(per[dom], 4)},
    }
    if a.cpu_tokens > 0:   # the oracle on a bounded sample of rows
        from oracle import fast_kernels as F
        rows = 512
        t0 = time.perf_counter()
        x64 = X[:rows].float().cpu().double().numpy()
        Yr, r = F.rms_layernorm_fwd(x64, w.float().cpu().double().numpy(), eps, gemma)
        F.rms_layernorm_bwd(dY[:rows].float().cpu().double().numpy(), x64, r, w.float().cpu().double().numpy(), gemma)
        p_np = pos[:rows].cpu().numpy()
        for t in (q, k):
            t64 = t[:rows].float().cpu().double().numpy()
            F.rope_bwd(F.rope_fwd(t64, p_np, 10000.0), p_np, 10000.0)
        l64 = logits[:rows].float().cpu().double().numpy()
        loss, ce, lse, n = F.cross_entropy_fwd(l64, lab_np[:rows])
        F.cross_entropy_bwd(l64, lab_np[:rows], lse, n)
        t = time.perf_counter() - t0
        model, nproc = host_cpu()
        out["cpu_baseline"] = {"value": round(total * rows / m / t / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle", "cpu_model": model, "nproc": nproc,
                               "sample": f"{rows} of {m} tokens, fp64 numpy (device-to-host copies included)",
                               "seconds": round(t, 3)}
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); "
              "the multi-GPU data-parallel design is described, not built.", file=sys.stderr)
        sys.exit(2)

    if a.workload == QUANT_WORKLOAD:
        bench_quantize(a)
        return
    if a.workload in FAST_WORKLOADS:
        bench_fast(a)
        return

    import torch

    import qlora_fine_tuning_amd as Q
    from qlora_fine_tuning_amd import _lib
    from qlora_fine_tuning_amd import inputs as I

    import dataclasses

    qkv = a.workload in QKV_WORKLOADS
    lin = a.workload in LINEAR_WORKLOADS
    cfg = {"llama7b_mlp": I.LLAMA_MLP, "mistral7b_mlp": I.MISTRAL_MLP,
           "gemma7b_mlp": I.GEMMA_MLP, "mistral7b_qkv": I.MISTRAL_QKV,
           "llama7b_qkv": I.LLAMA_QKV, "llama7b_q_proj": I.QPROJ,
           "mistral7b_kv_proj": I.MISTRAL_KV}[a.workload]
    full_m, full_r = cfg.m, cfg.r
    if a.tokens:
        cfg = dataclasses.replace(cfg, m=a.tokens)
    if a.rank:
        if not 1 <= a.rank <= 64:
            sys.exit("--rank must be in 1..64")
        cfg = dataclasses.replace(cfg, r=a.rank)
    dev = "cuda:0"
    w16 = a.base == "bf16"
    if lin:
        if w16:
            sys.exit("the linear workloads run the NF4 layer (--base nf4)")
        d = I.linear_inputs(cfg, dense_w=False, role="k" if a.workload == "mistral7b_kv_proj" else "")
        wl = Q.NF4Weight(d["codes"].to(dev), d["absmax"].to(dev))
        A_, B_ = d["A"].to(dev), d["B"].to(dev)
        X, dY = d["X"].to(dev), d["dY"].to(dev)
        nbytes = Q.linear_workspace_bytes(cfg.m, cfg.k, cfg.n, cfg.r, a.mode)
        w = wl
    elif qkv:
        if a.mode == "fused":
            sys.exit("the q/k/v path always stages its bf16 weights (no fused mode)")
        d = I.qkv_inputs(cfg, dense_w=w16)
        lora = [d[k + p].to(dev) for p in "qkv" for k in ("A", "B")]
        if w16:
            w = Q.Qkv16Weights(*(d["W" + p].to(dev) for p in "qkv"), *lora, s=cfg.s)
        else:
            nf = lambda p: Q.NF4Weight(d["W" + p + "_codes"].to(dev), d["W" + p + "_absmax"].to(dev))  # noqa: E731
            w = Q.QkvWeights(nf("q"), nf("k"), nf("v"), *lora, s=cfg.s)
        ns = (cfg.n_q, cfg.n_k, cfg.n_v)
        nbytes = Q.qkv_workspace_bytes(cfg.m, cfg.d, *ns, cfg.r)
        X = d["X"].to(dev)
        dYs = [d["dY" + p].to(dev) for p in "qkv"]
        dY = None
    else:
        d = I.mlp_inputs(cfg, dense_w=w16)
        lora = [d[k].to(dev) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")]
        if w16:
            w = Q.Mlp16Weights(d["Wg"].to(dev), d["Wu"].to(dev), d["Wd"].to(dev), *lora, s=cfg.s,
                               act=cfg.act)
            nbytes = Q.mlp16_workspace_bytes(cfg.m, cfg.d, cfg.h, cfg.r)
        else:
            nf = lambda wn: Q.NF4Weight(d[wn + "_codes"].to(dev), d[wn + "_absmax"].to(dev))  # noqa: E731
            w = Q.MlpWeights(nf("Wg"), nf("Wu"), nf("Wd"), *lora, s=cfg.s, act=cfg.act)
            nbytes = Q.mlp_workspace_bytes(cfg.m, cfg.d, cfg.h, cfg.r, a.mode)
        X, dY = d["X"].to(dev), d["dY"].to(dev)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step():
        if lin:
            _, U = Q.linear_fwd(X, wl, A_, B_, cfg.s, mode=a.mode, ws=ws)
            Q.linear_bwd(dY, X, U, wl, A_, B_, cfg.s, mode=a.mode, ws=ws)
        elif qkv:
            fwd, bwd = (Q.qkv16_fwd, Q.qkv16_bwd) if w16 else (Q.qkv_fwd, Q.qkv_bwd)
            _, _, _, U = fwd(X, w, ws=ws)
            bwd(*dYs, X, U, w, ws=ws)
        elif w16:
            _, sv = Q.mlp16_fwd(X, w, ws=ws)
            Q.mlp16_bwd(dY, X, sv, w, ws=ws)
        else:
            _, sv = Q.mlp_fwd(X, w, mode=a.mode, ws=ws)
            Q.mlp_bwd(dY, X, sv, w, mode=a.mode, ws=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    Q.trace_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / a.steps
    launches, gemm_ms, gemm_flops = Q.trace_read()
    Q.trace_enable(False)
    # per-step median and minimum: a second pass of the same steps with an
    # event at every step boundary (kept out of the timed region above, so
    # those events do not add to `value`)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(a.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps))
    step_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])

    peak_meas, shader_ghz = Q.probe_mfma_peak(20000)

    if lin:
        flops = linear_flops(cfg.m, cfg.k, cfg.n, cfg.r)
    elif qkv:
        flops = qkv_flops(cfg.m, cfg.d, ns, cfg.r)
    else:
        flops = mlp_flops(cfg.m, cfg.d, cfg.h, cfg.r)
    tflops = flops / (ms / 1e3) / 1e12
    achieved = gemm_flops / (gemm_ms / 1e3) / 1e12
    traffic = None if (w16 or cfg.m != full_m or cfg.r != full_r) else gemm_traffic(
        os.path.join(os.path.dirname(_lib.__file__), "csrc"), cfg.name,
        "staged" if (qkv or a.mode == "auto") else a.mode)
    if lin:
        metric = f"QLoRA linear fwd+bwd TFLOP/s + % bf16 MFMA peak, {cfg.name}, {cfg.m} tok"
        shape = {"k": cfg.k, "n": cfg.n}
    elif qkv:
        metric = METRIC_QKV.format(model="Mistral-7B" if a.workload == "mistral7b_qkv" else "Llama-7B")
        shape = {"d": cfg.d, "n_q": cfg.n_q, "n_k": cfg.n_k, "n_v": cfg.n_v}
    else:
        metric = METRIC
        shape = {"d": cfg.d, "h": cfg.h, "act": cfg.act}
    metric = metric.replace("8192 tok", f"{cfg.m} tok")
    out = {
        "metric": metric, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.m, **shape, "r": cfg.r, "s": cfg.s,
                   "weights": "bf16 (16-bit LoRA)" if w16 else "nf4 blocksize 64, fp32 absmax",
                   "dequant_mode": "none" if w16 else ("staged" if qkv else a.mode),
                   "global_batch": cfg.m, "parallelism": "none (1 GPU)"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(cfg.m / (ms / 1e3), 1),
        "step_ms_median": round(step_median, 4), "step_ms_min": round(per_step[0], 4),
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel (base GEMMs, LoRA as K-extension)",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "launches_per_step": launches // a.steps,
                     "avg_launch_ms": round(gemm_ms / launches, 4),
                     "gemm_share_of_step": round(gemm_ms / a.steps / ms, 4),
                     "measured_mfma_peak": round(peak_meas, 1),
                     "frac_of_measured_peak": round(achieved / peak_meas, 4),
                     "shader_ghz_under_mfma_load": round(shader_ghz, 3)},
    }
    if a.cpu_tokens > 0 and not w16 and not lin:
        del X, dY, ws, w
        torch.cuda.empty_cache()
        base = cpu_baseline_qkv if qkv else cpu_baseline
        out["cpu_baseline"] = base(cfg, d, min(a.cpu_tokens, cfg.m))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
