#!/usr/bin/env python3
"""Benchmark of one tensor-parallel layer shard, forward + backward, on one MI355X.

Workload (default): the GPT-2 8.3B-shape layer, one t = 8 shard (shard 0):
batch 8 x seq 1024 tokens, hidden 3072, 32 heads (4 per shard, d = 96), FFN 12288
(1536 per shard), causal, bf16 with fp32 accumulation; synthetic seeded inputs.
One step = MLP forward, attention forward, MLP backward, attention backward of
the shard through the C ABI, with inputs already resident in HBM.

Prints ONE JSON line on stdout:
  value            whole-job throughput, algorithmic TFLOP/s (2*M*N*K per GEMM,
                   causal-halved attention, no recompute counted)
  roofline         the dominant kernel's algorithmic TFLOP/s against the bf16
                   dense MFMA peak, timed live with HIP events on its stream
  cpu_baseline     the float64 CPU oracle timed on this host on a bounded sample
                   of the same workload (a baseline, not a target)
  step_spread      median / min of single steps (an event pair around each), warm and
                   with a 512 MiB write before each step (cold Infinity Cache)
  kernels          per-step breakdown (average duration, TFLOP/s or GB/s)
  other_workloads  the other per-shard shapes of the pages' models (BERT 3.9B t=8, 30B
                   t=4 and t=1), each timed in the same run before the headline
                   workload (its own warm-up and timed steps), ms/step and TFLOP/s
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shard-layer fwd+bwd TFLOP/s and % of bf16 MFMA peak, 8.3B-shape t=8 shard"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense); fp16 has the same peak
PEAK_HBM_GBS = 8000.0
# HBM bytes per step launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (copy-calibrated),
# valid while the kernel sources hash to the value recorded in the file
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_per_step_gpt8b_t8.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_costs(cfg):
    """Algorithmic FLOPs and minimum HBM bytes of each hook step (one launch each)."""
    from tensor_transformer_layer_02_amd.configs import causal_pairs
    T, h, Fs, w, d = cfg.tokens, cfg.hidden, cfg.ffn_per_shard, cfg.attn_width, cfg.head_dim
    e = 2
    pairs = cfg.batch * cfg.heads_per_shard * causal_pairs(cfg.seq, cfg.causal)
    g = lambda m, n, k: 2 * m * n * k
    # bytes: operands read once + outputs written once
    return {
        "MLP_UP": (g(T, Fs, h), (T * h + h * Fs + 2 * T * Fs) * e),
        "MLP_DOWN": (g(T, h, Fs), (T * Fs + Fs * h + T * h) * e),
        "QKV": (g(T, 3 * w, h), (T * h + 3 * h * w + 3 * T * w) * e),
        "ATTN_CORE": (2 * 2 * d * pairs, 4 * T * w * e + cfg.batch * cfg.heads_per_shard * cfg.seq * 4),
        "ATTN_OUT": (g(T, h, w), (T * w + w * h + T * h) * e),
        "MLP_DU": (g(T, Fs, h), (T * h + Fs * h + 2 * T * Fs) * e),
        "MLP_DW": (g(Fs, h, T) + g(h, Fs, T), (2 * T * Fs + 2 * T * h) * e + 2 * Fs * h * 4),
        "MLP_DB1": (0, T * Fs * e + Fs * 4),
        "MLP_DX": (g(T, h, Fs), (T * Fs + h * Fs + T * h) * e),
        "ATTN_DO": (g(T, w, h), (T * h + w * h + T * w) * e),
        "ATTN_CORE_BWD": (4 * 2 * d * pairs, 9 * T * w * e),
        # dW{q,k,v} and dWo share one launch
        "ATTN_DW": (g(h, 3 * w, T) + g(w, h, T), (T * h + 3 * T * w + T * w + T * h) * e + 4 * h * w * 4),
        "ATTN_DBIAS": (0, 3 * T * w * e + 3 * w * 4),
        "ATTN_DX": (g(T, h, 3 * w), (3 * T * w + 3 * w * h + T * h) * e),
    }


def peak_clock_mhz():
    """hipDeviceAttributeClockRate of device 0 (kHz in HIP) in MHz, from the runtime torch loaded."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    v = ctypes.c_int(0)
    HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5
    if hip.hipDeviceGetAttribute(ctypes.byref(v), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE, 0) != 0:
        return None
    return v.value // 1000


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same soname), created without
    the system-scope fence (hipEventDisableSystemFence): a record then only timestamps, instead of
    also writing back and invalidating the caches between the kernels it brackets."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev[i] = h
        self.n = n

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.ev[i])


def cpu_baseline(cfg, inp, nseq):
    """The float64 oracle, as it stands, on the first `nseq` sequences of the same inputs."""
    import oracle
    from tensor_transformer_layer_02_amd.configs import shard_flops
    from tensor_transformer_layer_02_amd.inputs import as_f64
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    sub = cfg.with_(batch=nseq)
    rows = sub.tokens
    p = {k: as_f64(v) for k, v in inp.items()}
    p["X"] = p["X"][:rows].copy()
    p["dZ"] = p["dZ"][:rows].copy()
    d = sub.dims()
    args = [p[n] for n in ("X", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo")]
    t0 = time.perf_counter()
    oracle.mlp_shard_fwd(d, 0, cfg.degree, p["X"], p["A"], p["b1"], p["B"])
    oracle.attn_shard_fwd(d, 0, cfg.degree, *args)
    oracle.mlp_shard_bwd(d, 0, cfg.degree, p["X"], p["A"], p["b1"], p["B"], p["dZ"])
    oracle.attn_shard_bwd(d, 0, cfg.degree, *args, p["dZ"])
    dt = time.perf_counter() - t0
    fl = shard_flops(sub, backward=True)["total"]
    what = (f"the whole workload ({cfg.batch} sequences, {rows} tokens" if nseq == cfg.batch else
            f"the first {nseq} of {cfg.batch} sequences ({rows} of {cfg.tokens} tokens")
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"shard 0 fwd+bwd on {what}; {fl / 1e9:.1f} GFLOP algorithmic), float64 C loops "
                      f"with OpenMP"}


# Other per-shard shapes of the pages' models, timed in the same run as the headline:
# (config, warm-up steps, timed steps), each about 0.05-0.3 s of GPU time.
OTHER_WORKLOADS = [("g30b_t4", 5, 10), ("g30b_t1", 3, 5), ("bert4b", 30, 20)]  # the closest to the headline last


def time_workload(name, dtype, W, K, keep=False):
    """ms per shard fwd+bwd step (HIP events around K steps after W warm-up steps, inputs resident)
    and algorithmic TFLOP/s of one other workload, shard 0.  With `keep` the workload's buffers are
    returned instead of freed, so that no free idles the GPU before the caller's next launches."""
    import torch

    from tensor_transformer_layer_02_amd.configs import CONFIGS, shard_flops
    from tensor_transformer_layer_02_amd.inputs import make_inputs
    from tensor_transformer_layer_02_amd.shard import ShardRun
    cfg = CONFIGS[name].with_(backward=True, dtype=dtype)
    run = ShardRun(cfg, make_inputs(cfg), shards=[0])
    for _ in range(W):
        run.step(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        run.step(0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    fl = shard_flops(cfg, backward=True)["total"]
    if not keep:
        del run
        torch.cuda.empty_cache()
        run = None
    tf = fl / (ms * 1e-3) / 1e12
    res = {"workload": f"{cfg.name}: {cfg.note}", "tokens": cfg.tokens, "hidden": cfg.hidden, "heads": cfg.heads,
            "ffn": cfg.ffn, "degree": cfg.degree, "causal": cfg.causal, "steps": K, "warmup": W,
            "ms_per_step": round(ms, 4), "flops_per_step": fl, "tflops": round(tf, 1),
            "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    return (res, run) if keep else res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first: after idle the GPU needs ~25 steps (~25 ms of load) to reach "
                         "its steady clock; per-step times fall from ~1.1 ms to ~0.925 ms over them")
    ap.add_argument("--config", default="gpt8b")
    ap.add_argument("--shard", type=int, default=0)
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default="bf16",
                    help="16-bit storage format (fp16: IEEE half with fp16 MFMAs; same dense peak)")
    ap.add_argument("--cpu-seqs", type=int, default=None,
                    help="sequences in the CPU-oracle sample (default: all of the workload's sequences)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other model shapes (BERT 3.9B t=8, 30B t=4 and t=1 shards), which are "
                         "otherwise timed first, in the same run, and reported under other_workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--recompute", action="store_true",
                    help="backward with activation recompute (the forward's activations rebuilt from X; "
                         "recompute FLOPs are not counted)")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole pre-LN layer instead (all t shards of both sublayers plus the "
                         "residual / LayerNorm kernels, on one GPU) and print its own JSON line")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor library (hipBLASLt through torch.matmul, plain GEMMs with "
                         "contiguous operands, 16-bit outputs, no epilogues) on the GEMM shapes of the "
                         "step, for context, and print one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's shard; runs on more than one GPU "
                                   "are not supported (the cross-shard all-reduce is out of scope)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from tensor_transformer_layer_02_amd import tpshard as tp
    from tensor_transformer_layer_02_amd.configs import CONFIGS, shard_flops
    from tensor_transformer_layer_02_amd.inputs import make_inputs
    from tensor_transformer_layer_02_amd.shard import ShardRun

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return
    cfg = CONFIGS[args.config]
    if not cfg.backward:
        cfg = cfg.with_(backward=True)
    if cfg.dtype != args.dtype and cfg.dtype != "fp32":
        cfg = cfg.with_(dtype=args.dtype)
    K, W = args.steps, args.warmup
    if args.vendor_gemm:
        return vendor_gemm(cfg, K, W)
    if args.layer:
        return bench_layer(cfg, K, W)
    log(f"[bench] {cfg.note}: T={cfg.tokens} h={cfg.hidden} F/t={cfg.ffn_per_shard} H/t={cfg.heads_per_shard} "
        f"d={cfg.head_dim} shard={args.shard}")
    inp = make_inputs(cfg)
    run = ShardRun(cfg, inp, shards=[args.shard], recompute=args.recompute)
    step = lambda: run.step(args.shard, recompute=args.recompute)
    flops = shard_flops(cfg, backward=True)["total"]
    prop = torch.cuda.get_device_properties(0)
    clock_mhz = peak_clock_mhz()
    log(f"[bench] device {prop.name} ({prop.gcnArchName}) CUs={prop.multi_processor_count} peak clock "
        f"{clock_mhz} MHz, peak(bf16 dense)={PEAK_BF16_TFLOPS} TFLOP/s")

    if not args.no_kernel_timing:
        ev = HipEvents(2 * len(tp.STEPS) * K)  # for the per-kernel pass below
    # ---- the other model shapes first (same run; the headline below keeps its own W and K).  The
    # headline's buffers already exist and the last workload's are kept until the process ends (a
    # free would idle the GPU), so its W warm-up steps follow that workload's steps with the GPU
    # kept busy: after even 20 ms of idle the clocks boost, overshoot and settle over ~30 steps,
    # which a short warm-up would otherwise measure instead of the steady state.
    others, held = [], None
    if not args.no_others and args.config == "gpt8b" and not args.recompute:
        for i, (name, ow, ok) in enumerate(OTHER_WORKLOADS):
            last = i + 1 == len(OTHER_WORKLOADS)
            r = time_workload(name, cfg.dtype, ow, ok, keep=last)
            if last:
                r, held = r
            others.append(r)
            log(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step  {r['tflops']} TFLOP/s  "
                f"({r['pct_of_bf16_peak']}% of bf16 peak)")

    for _ in range(W):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps on the current stream ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / K
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.4f} ms/step  {tflops:.1f} TFLOP/s  ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)"
        f"  wall {wall:.3f}s")

    # ---- spread over single steps (an event pair around each), then a cold-cache figure:
    # a 512 MiB write (twice the 256 MB Infinity Cache) before each step evicts weights and inputs
    def single_steps(n, before=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            if before is not None:
                before()
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    def median(v):
        n = len(v)
        return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])

    warm = single_steps(K)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = single_steps(min(K, 10), before=lambda: scratch.fill_(1))
    del scratch
    spread = {"warm_median_ms": round(median(warm), 5), "warm_min_ms": round(warm[0], 5),
              "cold_median_ms": round(median(cold), 5), "cold_min_ms": round(cold[0], 5),
              "cold_tflops": round(flops / (median(cold) * 1e-3) / 1e12, 2), "cold_steps": len(cold),
              "note": "event pair around each single step; cold: 512 MiB written before each step"}
    log(f"[bench] single steps: warm median {spread['warm_median_ms']:.4f} ms (min {spread['warm_min_ms']:.4f}), "
        f"cold-cache median {spread['cold_median_ms']:.4f} ms ({spread['cold_tflops']} TFLOP/s)")

    # ---- per-kernel timing: HIP event pairs around each step's launch, same stream.  The events
    # exist already (creating hundreds of them here would leave the GPU idle), and a few untimed
    # steps first keep this pass at the same steady clock as the timed region.
    kernels, roof = [], None
    if not args.no_kernel_timing:
        nst = len(tp.STEPS)
        for _ in range(10):
            step()
        tp.tp_profile_enable(ev.ev, K)
        e0.record()
        for _ in range(K):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms_hooked = e0.elapsed_time(e1) / K
        counts = [tp.tp_profile_count(s) for s in range(nst)]
        nkern = [tp.tp_profile_kernels(s) for s in range(nst)]
        tp.tp_profile_enable(None, 0)
        costs = step_costs(cfg)
        for s, name in enumerate(tp.STEPS):
            n = min(counts[s], K)
            if n == 0:
                continue
            durs = [ev.elapsed_ms(2 * (s * K + k), 2 * (s * K + k) + 1) for k in range(n)]
            avg = sum(durs) / n
            fl, by = costs[name]
            kernels.append({"step": name, "avg_us": round(avg * 1e3, 2), "launches": n,
                            "kernels_per_launch": round(nkern[s] / counts[s], 3),
                            "tflops": round(fl / (avg * 1e-3) / 1e12, 1) if fl else None,
                            "gbs": round(by / (avg * 1e-3) / 1e9, 1)})
        ev.close()
        tot = sum(k["avg_us"] for k in kernels)
        for k in kernels:
            k["share"] = round(k["avg_us"] / tot, 3)
        log(f"[bench] with per-step events: {ms_hooked:.4f} ms/step")
        for k in kernels:
            log(f"  {k['step']:<14} {k['avg_us']:9.2f} us  {k['share'] * 100:5.1f}%  "
                f"{(str(k['tflops']) + ' TF/s') if k['tflops'] else '':>14}  {k['gbs']:8.1f} GB/s")
        # the dominant kernel: the longest step that is exactly one kernel launch
        dom = max((k for k in kernels if k["kernels_per_launch"] == 1), key=lambda k: k["avg_us"])
        fl, by = costs[dom["step"]]
        ach = fl / (dom["avg_us"] * 1e-6) / 1e12
        traffic, tnote = None, "no counter table for this workload"
        if cfg.name == "gpt8b" and cfg.dtype == "bf16" and args.shard == 0:
            from tensor_transformer_layer_02_amd.profiling import read_traffic, source_hash
            tab, h = read_traffic(TRAFFIC_FILE)
            if h is None:
                tnote = "counter table missing"
            elif h != source_hash():
                tnote = "kernel sources changed since the counters were taken"
            elif dom["step"] in tab:
                traffic = int(round(sum(tab[dom["step"]])))
                tnote = (f"FETCH_SIZE+WRITE_SIZE bytes per launch (copy-calibrated), "
                         f"{os.path.relpath(TRAFFIC_FILE, ROOT)}; algorithmic minimum {by} bytes")
        roof = {"bound": "mfma", "kernel": dom["step"], "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_note": tnote, "flops_per_launch": fl, "avg_us": dom["avg_us"]}

    cpu = None
    if not args.no_cpu_baseline:
        nseq = cfg.batch if args.cpu_seqs is None else max(1, min(args.cpu_seqs, cfg.batch))
        log(f"[bench] CPU oracle baseline on {nseq} of {cfg.batch} sequence(s) ...")
        cpu = cpu_baseline(cfg, inp, nseq)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads ({cpu['seconds']} s)")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": f"{cfg.name}: {cfg.note}", "batch": cfg.batch, "seq": cfg.seq,
                   "tokens": cfg.tokens, "hidden": cfg.hidden, "heads": cfg.heads, "ffn": cfg.ffn,
                   "degree": cfg.degree, "shard": args.shard, "causal": cfg.causal,
                   "flops_per_step": flops,
                   "flops_per_step_dense_attention": shard_flops(cfg.with_(causal=False), backward=True)["total"],
                   "parallelism": "one tp shard on one GPU (no collectives)",
                   "activations": "recomputed in the backward" if args.recompute else "saved"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_spread": spread,
        "gpu": {"name": prop.name, "arch": prop.gcnArchName, "cus": prop.multi_processor_count,
                "peak_clock_mhz": clock_mhz},
        "kernels": kernels,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


def vendor_gemm(cfg, K, W):
    """The vendor GEMM (hipBLASLt via torch.matmul) on the shapes of each GEMM step of the shard,
    [M, K] x [K, N] with both operands contiguous and a 16-bit output (no bias, GeLU or fp32
    output): a context figure for the library's kernels, not part of the path."""
    import torch

    T, h, Fs, w = cfg.tokens, cfg.hidden, cfg.ffn_per_shard, cfg.attn_width
    dt = torch.float16 if cfg.dtype == "fp16" else torch.bfloat16
    steps = {  # step: list of (M, K, N)
        "MLP_UP": [(T, h, Fs)], "MLP_DOWN": [(T, Fs, h)], "QKV": [(T, h, 3 * w)], "ATTN_OUT": [(T, w, h)],
        "MLP_DU": [(T, h, Fs)], "MLP_DW": [(Fs, T, h), (h, T, Fs)], "MLP_DX": [(T, Fs, h)],
        "ATTN_DO": [(T, h, w)], "ATTN_DW": [(h, T, 3 * w)], "ATTN_DWO": [(w, T, h)], "ATTN_DX": [(T, 3 * w, h)],
    }
    gen = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for name, gemms in steps.items():
        ops = [(torch.randn((m, k), generator=gen, device="cuda", dtype=dt),
                torch.randn((k, n), generator=gen, device="cuda", dtype=dt)) for m, k, n in gemms]
        for _ in range(W):
            for a, b in ops:
                torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            for a, b in ops:
                torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / K * 1e3
        fl = sum(2 * m * k * n for m, k, n in gemms)
        rows.append({"step": name, "avg_us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 1)})
        log(f"  {name:<10} {us:9.2f} us  {rows[-1]['tflops']:8.1f} TF/s")
    print(json.dumps({"vendor_gemm": "hipBLASLt via torch.matmul", "dtype": cfg.dtype, "steps": K,
                      "warmup": W, "workload": cfg.name, "gemms": rows}), flush=True)


def bench_layer(cfg, K, W):
    """The whole pre-LN layer on one GPU: every shard of both sublayers, the fused residual-sum +
    LayerNorm kernels and the LayerNorm backward.  value = algorithmic TFLOP/s of the t shards;
    the roofline object is the LayerNorm / residual phase with the largest share (HBM-bound)."""
    import torch

    from tensor_transformer_layer_02_amd.configs import shard_flops
    from tensor_transformer_layer_02_amd.inputs import make_layer_inputs
    from tensor_transformer_layer_02_amd.layer import PreLNLayer

    log(f"[bench] pre-LN layer {cfg.name}: T={cfg.tokens} h={cfg.hidden} F={cfg.ffn} H={cfg.heads} "
        f"t={cfg.degree} shards on one GPU")
    layer = PreLNLayer(cfg, make_layer_inputs(cfg))
    flops = cfg.degree * shard_flops(cfg, backward=True)["total"]
    phases = PreLNLayer.FORWARD + PreLNLayer.BACKWARD
    for _ in range(W):
        layer.forward()
        layer.backward()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        layer.forward()
        layer.backward()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/layer step  {tflops:.1f} TFLOP/s  ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
    # per-phase timing (events on the current stream around each phase)
    ev = {ph: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for ph in phases}
    for k in range(K):
        for ph in phases:
            ev[ph][k][0].record()
            getattr(layer, ph)()
            ev[ph][k][1].record()
    torch.cuda.synchronize()
    nbytes = layer.ln_bytes()
    rows = []
    for ph in phases:
        us = sum(a.elapsed_time(b) for a, b in ev[ph]) / K * 1e3
        r = {"phase": ph, "avg_us": round(us, 2)}
        if ph in nbytes:
            r["bytes"] = nbytes[ph]
            r["gbs"] = round(nbytes[ph] / (us * 1e-6) / 1e9, 1)
        rows.append(r)
        log(f"  {ph:<14} {us:9.2f} us" + (f"  {r['gbs']:8.1f} GB/s" if "gbs" in r else ""))
    dom = max((r for r in rows if "gbs" in r), key=lambda r: r["avg_us"])
    out = {
        "metric": "pre-LN layer fwd+bwd TFLOP/s, all t shards on one GPU, 8.3B shape",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic", "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": f"{cfg.name} pre-LN layer: {cfg.degree} shards + residual/LayerNorm kernels",
                   "tokens": cfg.tokens, "hidden": cfg.hidden, "heads": cfg.heads, "ffn": cfg.ffn,
                   "degree": cfg.degree, "flops_per_step": flops},
        "roofline": {"bound": "hbm", "kernel": dom["phase"], "achieved": dom["gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dom["gbs"] / PEAK_HBM_GBS, 4), "traffic": None,
                     "traffic_note": "algorithmic bytes; no counter table for this workload"},
        "cpu_baseline": None,
        "phases": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
