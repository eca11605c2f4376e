"""Benchmark of the dual-phase policy step on one MI355X.

One step = one observation through the whole hot path: the bidirectional
prefix pass writing the K/V cache (vla_prefix_encode) and the flow-matching
action expert refining a noise chunk over T Euler steps (vla_denoise_chunk).
Workload: the single-camera bf16 policy (288 prefix tokens, 18 + 18 layers,
50 x 32 action chunk, 10 steps, batch 1) with seeded synthetic weights and
inputs, all resident in HBM before timing starts.

Prints one JSON line: action chunks/s, per-phase latency, the roofline of the
kernel with the largest share of GPU time (its launches timed with HIP events
in a separate probe pass after the timed region, so the timing does not
perturb the measured steps), a roofline entry per phase, and the CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0
PEAK_HBM_GBS = 8000.0

# HBM-side bytes from rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter
# reads for a plain copy of known size (profiles/hbm_bytes_denoise_single_camera_bf16.md).  Valid for the
# single-camera bf16 workload with the absorbed cross sublayer and the kernels as they were measured; None where no
# measurement stands.
ATTN_KERNEL = "k_attn_chunk<256>"
SCORES_KERNEL = "k_chunk<2, 1, 6, 8, true>"
SCORES_TRAFFIC_BYTES_PER_LAUNCH = 6356989  # the absorbed score product, per launch
GATEUP_KERNEL = "k_chunk<2, 4, 2, 8, true>"
GATEUP_TRAFFIC_BYTES_PER_LAUNCH = 31905253  # the expert gate/up product, per launch
ATTN_TRAFFIC_BYTES_PER_LAUNCH = 13895459   # mean over all launches of a bench run (prefix and expert self attention)
DENOISE_TRAFFIC_BYTES_PER_STEP = 1590477858  # every kernel of one solver step (the denoise graph's nodes)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=1, help="workload index (1 = single camera bf16)")
    p.add_argument("--attn", choices=("cross", "joint"), default="cross",
                   help="cache form: projected final states (cross) or per-layer prefix K/V (joint, the pi0 form)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-s", type=float, default=30.0)
    p.add_argument("--no-extras", action="store_true",
                   help="skip the solver-step sweep, the two-stream pipelined run and the ternary ablation")
    p.add_argument("--no-batched", action="store_true", help="skip the batched-workload entry")
    p.add_argument("--no-roofline", action="store_true",
                   help="skip the probe pass of the dominant kernel (for counter passes that must see only the "
                        "policy steps themselves)")
    p.add_argument("--pipelined", action="store_true",
                   help="also time the two-stream schedule (prefix of observation k+1 beside the solver of k); "
                        "it is slower than the serial one on this GPU and is left out of the default line")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB mebibytes (reference for the HBM byte counters) and exit")
    return p.parse_args()


def copy_calibration(mib):
    """One plain device-to-device copy of a known size: its FETCH_SIZE / WRITE_SIZE counters scale the kernels'."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)


def prefix_flops(c):
    """Algorithmic FLOPs of one prefix pass (+ cache projection) for one observation.  With joint
    attention the cache is the layers' own K/V: no projection, and the last layer stops at its K/V."""
    N = c.n_prefix
    qkv = 2 * N * c.d_p * (c.Hq + 2 * c.Hkv) * c.hd
    attn = 4 * N * N * c.Hq * c.hd
    o = 2 * N * c.Hq * c.hd * c.d_p
    mlp = 2 * N * c.d_p * 2 * c.F_p + 2 * N * c.F_p * c.d_p
    if c.attn == "joint":
        return c.L_p * qkv + (c.L_p - 1) * (attn + o + mlp)
    cache = 2 * N * c.d_p * c.L_e * 2 * c.Hkv_e * c.hd_e
    return c.L_p * (qkv + attn + o + mlp) + cache


def expert_step_flops(c):
    """Algorithmic FLOPs of one denoise step for the whole batch (the bound at the batched workload)."""
    qe, kve = c.Hq_e * c.hd_e, c.Hkv_e * c.hd_e
    M = c.batch * c.H
    cross = 0 if c.attn == "joint" else 2 * M * c.d_e * qe * 2 + 4 * M * c.n_prefix * qe
    keys = c.H + (c.n_prefix if c.attn == "joint" else 0)
    per_layer = (2 * M * c.d_e * (qe + 2 * kve) + 4 * M * keys * qe + 2 * M * qe * c.d_e + cross
                 + 2 * M * c.d_e * 2 * c.F_e + 2 * M * c.F_e * c.d_e)
    return c.L_e * per_layer + 2 * M * c.d_e * (c.d_a + c.d_a)


def expert_step_bytes(c, absorbed=False):
    """Algorithmic HBM bytes of one denoise step: every expert weight once (bf16) plus the cache.  With the
    absorbed cross sublayer a step reads each layer's Wq_j^T K^T and V Wo_j^T (Hq_e x n_prefix x d_e each)
    in place of the cross-attention query and output weights and the cached keys and values."""
    qe, kve = c.Hq_e * c.hd_e, c.Hkv_e * c.hd_e
    cross = 0 if c.attn == "joint" else qe * c.d_e + c.d_e * qe  # cross-attention query and output
    if absorbed:
        cross = 2 * c.Hq_e * c.n_prefix * c.d_e
    per_layer = (qe + 2 * kve) * c.d_e + c.d_e * qe + cross + 2 * c.F_e * c.d_e + c.d_e * c.F_e
    weights = c.L_e * per_layer + c.d_e * c.d_a * 2
    cache = 0 if absorbed else c.batch * c.L_e * 2 * kve * c.n_prefix
    return 2 * (weights + cache)


def absorbed_form(vla, model, c):
    """Whether this model's encode writes the absorbed cross-attention products (the cache storage then
    exceeds the keys, values and lengths, as vla.h states)."""
    if c.precision == "f32" or c.attn == "joint":
        return False
    np_ = (c.n_prefix + 31) // 32 * 32
    core = c.batch * c.L_e * 2 * c.Hkv_e * np_ * c.hd_e * 2
    plain = (core + 255) // 256 * 256 + (c.batch * 4 + 255) // 256 * 256
    return vla.vla_kv_cache_bytes(model, c.batch, c.n_prefix) > plain


SWEEP_STEPS = (1, 2, 4, 8, 16)


def solver_sweep(vla, model, zt, xt, kv_storage, reps=5):
    """Eq. 3 measured: latency with the cache (one prefix pass, then T solver steps) against re-encoding the
    prefix before every step, for T in SWEEP_STEPS, each the median of `reps` runs timed with the library's
    HIP events.  L(T) = P + T E is fitted to the cached latencies; `ideal_speedup` is T (P + E) / (P + T E)."""
    import torch
    xa = torch.empty_like(xt)
    xb = torch.empty_like(xt)
    cached, recompute = [], []
    for T in SWEEP_STEPS:
        c, r = [], []
        for _ in range(reps):
            kv, tp = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage, timing=True)
            _, td = vla.vla_denoise_chunk(model, kv, xt, T, out=xa, timing=True)
            kv.close()
            c.append(tp["prefix_ms"] + td["denoise_ms"])
            tot, x, y = 0.0, xt, xa
            for k in range(T):
                kv, tp = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage, timing=True)
                _, td = vla.vla_denoise_chunk(model, kv, x, 1, schedule=[k / T, (k + 1) / T], out=y, timing=True)
                kv.close()
                tot += tp["prefix_ms"] + td["denoise_ms"]
                x, y = y, (xb if y is xa else xa)
            r.append(tot)
        cached.append(float(np.median(c)))
        recompute.append(float(np.median(r)))
    Ts = np.array(SWEEP_STEPS, dtype=np.float64)
    E, P = np.polyfit(Ts, np.array(cached), 1)
    return {"T": list(SWEEP_STEPS), "cached_ms": cached, "recompute_ms": recompute,
            "speedup": [r / c for r, c in zip(recompute, cached)],
            "fit": {"P_ms": float(P), "E_ms": float(E)},
            "ideal_speedup": [float(T * (P + E) / (P + T * E)) for T in Ts]}


W2A8_SHAPES = ((320, 7680, 2560), (320, 2560, 2560), (320, 13824, 2560), (320, 2560, 6912))


def w2a8_ablation(vla, reps=5):
    """The page's ternary-kernel comparison restated on CDNA4: the int8 matrix-core kernel the ternary
    prefix uses against a vector-ALU kernel on v_dot4_i32_i8 (the dp4a counterpart), at the ternary
    workload's four projection shapes (320 rows), each the median kernel time of `reps` calls."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(7)
    out = []
    for M, N, K in W2A8_SHAPES:
        a = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int8).cuda()
        alpha = torch.rand(M, generator=g).cuda() * 0.01
        packed = torch.randint(0, 255, (N, K // 4), generator=g, dtype=torch.uint8)
        packed = (packed & 0x55).cuda()  # codes 0 and 1 only: valid ternary bytes
        row = {"M": M, "N": N, "K": K}
        for name, path in (("mfma", vla.W2A8_MFMA), ("dot4", vla.W2A8_DOT4)):
            ts = [vla.vla_w2a8_gemm_ex(a, alpha, packed, [0.02], N, path, want_acc=False, timing=True)[2]
                  for _ in range(reps)]
            ms = float(np.median(ts))
            row[name + "_us"] = ms * 1e3
            row[name + "_tops"] = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        row["speedup"] = row["dot4_us"] / row["mfma_us"]
        out.append(row)
    return out


def pipelined(vla, model, cfg, zt, xt, n, warmup=2):
    """Observations back to back with the prefix pass of observation k + 1 on a second stream while the solver
    of observation k runs (two cache buffers).  Returns chunks/s over n observations; every output is the same
    as the serial run's (the test suite checks that bit for bit)."""
    import torch
    nbytes = vla.vla_kv_cache_bytes(model, cfg.batch, cfg.n_prefix)
    store = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty(xt.shape, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    sp, sd = torch.cuda.Stream(), torch.cuda.Stream()
    enc = [torch.cuda.Event() for _ in range(2)]
    dec = [torch.cuda.Event() for _ in range(2)]

    def run(count):
        kvs = [None, None]
        kvs[0] = vla.vla_prefix_encode(model, zt, kv_storage=store[0], stream=sp)
        enc[0].record(sp)
        for k in range(count):
            b = k % 2
            if k + 1 < count:
                nb = 1 - b
                if k >= 1:
                    sp.wait_event(dec[nb])  # the solver of observation k - 1 has read that cache
                    kvs[nb].close()
                kvs[nb] = vla.vla_prefix_encode(model, zt, kv_storage=store[nb], stream=sp)
                enc[nb].record(sp)
            sd.wait_event(enc[b])
            vla.vla_denoise_chunk(model, kvs[b], xt, cfg.steps, out=outs[b], stream=sd)
            dec[b].record(sd)
        torch.cuda.synchronize()
        for kv in kvs:
            if kv is not None:
                kv.close()

    run(warmup)
    t0 = time.perf_counter()
    run(n)
    el = time.perf_counter() - t0
    return {"value": cfg.batch * n / el, "unit": "chunks/s", "observations": n,
            "note": "prefix of observation k+1 overlapped with the solver of observation k on two streams"}


DTYPE = {"f32": "f32", "bf16": "bf16", "w2a8": "int8 x ternary (int32 accumulation) prefix, bf16 expert"}


def attn_launch_bytes(c):
    """Algorithmic bytes of one launch of the chunk attention kernel, per class: queries and keys / values
    read once, the output written once (bf16).  Prefix: the encode's bidirectional attention (cross form);
    self: the expert's attention over the chunk (joint: plus prefix layer e's keys and values); cross: the
    expert's attention into the cached block of one layer."""
    N, M = c.batch * c.n_prefix, c.batch * c.H
    qp, kvp = c.Hq * c.hd, c.Hkv * c.hd
    qe, kve = c.Hq_e * c.hd_e, c.Hkv_e * c.hd_e
    joint_kv = 2 * N * kve if c.attn == "joint" else 0
    return {"prefix": 2 * (2 * N * qp + 2 * N * kvp),
            "self": 2 * (2 * M * qe + 2 * M * kve + joint_kv),
            "cross": 2 * (2 * M * qe + 2 * N * kve)}


PROBE_REPEAT = 20


def probe_mean_ms(vla, model, kind, run):
    """Mean device time of one launch of a kernel class during run(): each launch of the class is issued
    PROBE_REPEAT times back to back between two HIP events, so the events' own cost is spread thin (graphs
    off for the run: a probe sees only launches outside a captured graph; the run's results are discarded)."""
    import torch
    prev = os.environ.get("VLA_NO_GRAPH")
    os.environ["VLA_NO_GRAPH"] = "1"
    try:
        probe = vla.Probe(model, kind, repeat=PROBE_REPEAT)
        run()
        torch.cuda.synchronize()
        ms, n = probe.collect()
    finally:
        if prev is None:
            os.environ.pop("VLA_NO_GRAPH", None)
        else:
            os.environ["VLA_NO_GRAPH"] = prev
    return (ms / n if n else None), n


def scores_launch_bytes(c):
    """Algorithmic bytes of one launch of the absorbed score product: its weights Wq_j^T K^T (Hq_e x n_prefix
    rows of d_e, bf16) and the normalised chunk rows read once, the bf16 block weights and the fp32 block
    statistics (max, sum per row and 32-key block) written once."""
    M, S = c.batch * c.H, c.Hq_e * c.n_prefix
    return 2 * S * c.d_e + 2 * M * c.d_e + 2 * M * S + 8 * M * (S // 32)


def gateup_launch_bytes(c):
    """Algorithmic bytes of one launch of the expert's gate/up product: its 2 F_e x d_e bf16 weights and the
    chunk rows read once, the GeGLU output (F_e per row, bf16) written once."""
    M = c.batch * c.H
    return 2 * (2 * c.F_e * c.d_e) + 2 * M * c.d_e + 2 * M * c.F_e


def dominant_kernel_roofline(vla, model, cfg, zt, xt, out, kv_storage, absorbed=False):
    """Roofline of the kernel with the largest share of GPU time in the committed traces: the chunk
    attention kernel for the bf16 workloads (prefix attention in the encode, self and cross attention in
    every solver step), the int8 ternary GEMM for the ternary one.  Achieved = algorithmic bytes (or
    operations) of one policy step's launches of that kernel over their summed mean durations, the
    durations probed per class after the timed region."""
    L_p, T, L_e = cfg.L_p, cfg.steps, cfg.L_e

    def encode():
        kv = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage)
        kv.close()

    def denoise():
        kv = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage)
        vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out=out)
        kv.close()

    if cfg.precision == "w2a8":
        N = cfg.batch * cfg.n_prefix
        qw, qkvw = cfg.Hq * cfg.hd, (cfg.Hq + 2 * cfg.Hkv) * cfg.hd
        shapes = {vla.PROBE_PREFIX_QKV: (qkvw, cfg.d_p), vla.PROBE_PREFIX_O: (cfg.d_p, qw),
                  vla.PROBE_PREFIX_GATEUP: (2 * cfg.F_p, cfg.d_p), vla.PROBE_PREFIX_DOWN: (cfg.d_p, cfg.F_p)}
        ops = t = 0.0
        per = {}
        for kind, (n_out, k_in) in shapes.items():
            ms, n = probe_mean_ms(vla, model, kind, encode)
            if ms is None:
                return None
            o = 2.0 * N * n_out * k_in
            per[f"{n_out}x{k_in}"] = {"us": ms * 1e3, "tops": o / (ms * 1e-3) / 1e12}
            ops += L_p * o
            t += L_p * ms
        tops = ops / (t * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": tops / PEAK_INT8_TOPS, "traffic": None, "kernel": "k_gemm_w2a8 (int8 x ternary prefix GEMMs)",
                "avg_launch_us": t * 1e3 / (4 * L_p), "launches_per_step": 4 * L_p, "ops_per_step": ops,
                "per_shape": per, "timing": f"HIP events around {PROBE_REPEAT} back-to-back repeats of each launch, separate probe pass after the timed region, graphs off"}
    if cfg.precision != "bf16":
        return None
    attention = attention_roofline(vla, model, cfg, encode, denoise, absorbed)
    if not absorbed:
        return attention
    timing = (f"HIP events around {PROBE_REPEAT} back-to-back repeats of each launch, separate probe pass after "
              "the timed region, graphs off")
    measured = cfg.name == "single_camera_bf16"

    def entry(kind, nb, kernel, traffic):
        ms, n = probe_mean_ms(vla, model, kind, denoise)
        if ms is None:
            return None
        gbs = nb / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": traffic if measured else None, "kernel": kernel, "avg_launch_us": ms * 1e3,
                "bytes_per_launch": nb, "launches_per_step": T * L_e, "timing": timing}

    # with the absorbed cross sublayer the expert's gate/up product is the largest share of the trace
    top = entry(vla.PROBE_EXPERT_GATEUP, gateup_launch_bytes(cfg),
                GATEUP_KERNEL + " (action-expert gate/up product with the GeGLU epilogue)", GATEUP_TRAFFIC_BYTES_PER_LAUNCH)
    if top is None:
        return None
    top["scores"] = entry(vla.PROBE_EXPERT_SCORES, scores_launch_bytes(cfg),
                          SCORES_KERNEL + " (absorbed cross sublayer: score product with block max and sums)",
                          SCORES_TRAFFIC_BYTES_PER_LAUNCH)
    top["attention"] = attention
    return top


def attention_roofline(vla, model, cfg, encode, denoise, absorbed):
    """The chunk attention kernel over one policy step's launches (prefix, expert self, and expert cross
    unless the cross sublayer is absorbed)."""
    L_p, T, L_e = cfg.L_p, cfg.steps, cfg.L_e
    b = attn_launch_bytes(cfg)
    classes = [("prefix", vla.PROBE_PREFIX_ATTN, encode, L_p), ("self", vla.PROBE_EXPERT_SELF_ATTN, denoise, T * L_e)]
    if cfg.attn == "cross":
        classes.append(("cross", vla.PROBE_EXPERT_CROSS_ATTN, denoise, T * L_e))
    tot_b = tot_t = 0.0
    launches = 0
    per = {}
    for name, kind, run, count in classes:
        ms, n = probe_mean_ms(vla, model, kind, run)
        if ms is None and name == "cross":
            continue  # the absorbed cross sublayer runs no attention over the cache
        if ms is None:
            return None
        per[name] = {"us": ms * 1e3, "bytes": b[name], "gbs": b[name] / (ms * 1e-3) / 1e9, "launches_per_step": count}
        tot_b += count * b[name]
        tot_t += count * ms
        launches += count
    gbs = tot_b / (tot_t * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": ATTN_TRAFFIC_BYTES_PER_LAUNCH if (cfg.name == "single_camera_bf16" and absorbed) else None,
            "kernel": ATTN_KERNEL + " (chunk attention: " + ", ".join(per) + ")",
            "avg_launch_us": tot_t * 1e3 / launches, "bytes_per_launch": tot_b / launches,
            "launches_per_step": launches, "per_class": per,
            "timing": f"HIP events around {PROBE_REPEAT} back-to-back repeats of each launch, separate probe pass after the timed region, graphs off"}


def batched_entry(vla, model, cfg1, steps=3, warmup=1):
    """The batched workload (16 observations of 512 prefix tokens, 800 chunk rows, 10 solver steps): the
    same model shapes as the single-camera workload, so the line's own model times it on its own seeded
    16 x 512 prefixes and noise.  At 800 rows the expert's products are bound by the MFMA peak."""
    import torch
    import synth
    cfg = synth.config(3)
    assert (cfg.d_p, cfg.L_p, cfg.d_e, cfg.L_e, cfg.F_p, cfg.F_e) == (cfg1.d_p, cfg1.L_p, cfg1.d_e, cfg1.L_e,
                                                                       cfg1.F_p, cfg1.F_e)
    zt = torch.from_numpy(synth.make_prefix(cfg, 3)).cuda()
    xt = torch.from_numpy(synth.make_noise(cfg, 3)).cuda()
    out = torch.empty(xt.shape, dtype=torch.bfloat16, device="cuda")
    store = torch.empty(vla.vla_kv_cache_bytes(model, cfg.batch, cfg.n_prefix), dtype=torch.uint8, device="cuda")

    def step():
        kv = vla.vla_prefix_encode(model, zt, kv_storage=store)
        vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out=out)
        kv.close()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    kv, tp = vla.vla_prefix_encode(model, zt, kv_storage=store, timing=True)
    _, td = vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out=out, timing=True)
    kv.close()
    pf, ef = prefix_flops(cfg) * cfg.batch, expert_step_flops(cfg)
    return {"value": cfg.batch * steps / el, "unit": "chunks/s", "steps": steps,
            "workload": f"{cfg.name}: {cfg.batch} observations x {cfg.n_prefix} prefix tokens, "
                        f"{cfg.batch * cfg.H} chunk rows, {cfg.steps} solver steps (this line's model weights)",
            "prefix_ms": tp["prefix_ms"], "denoise_ms": td["denoise_ms"], "denoise_step_ms": td["step_ms"],
            "prefix_mfma_frac": pf / (tp["prefix_ms"] * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
            "denoise_mfma_frac": ef / (td["step_ms"] * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
            "denoise_hbm_frac": expert_step_bytes(cfg) / (td["step_ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9),
            "denoise_bound": "mfma"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs the policy step on one GPU: --gpus must be 1"}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import synth
    from prefix_cache_flow_amd import vla

    torch.cuda.set_device(0)
    cfg = synth.config(args.config)
    if args.attn == "joint":
        cfg = synth.config(args.config, attn="joint", name=cfg.name.replace("_bf16", "") + "_joint_bf16")
    t0 = time.time()
    w, betas = synth.make_weights(cfg, args.config)
    z0 = synth.make_prefix(cfg, args.config)
    x0 = synth.make_noise(cfg, args.config)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    names = [n for n, _, _ in synth.weight_specs(cfg)]
    tensors = vla.upload_weights(cfg.to_dict(), [w[n] for n in names])
    bl = [betas[n] for n, _, k in synth.weight_specs(cfg) if k == "ternary"] or None
    model = vla.vla_model_create(cfg.to_dict(), tensors, bl)
    del tensors
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"# model built at {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    zt = torch.from_numpy(z0).cuda()
    xt = torch.from_numpy(x0).cuda()
    out = torch.empty(x0.shape, dtype=torch.bfloat16, device="cuda")
    kv_storage = torch.empty(vla.vla_kv_cache_bytes(model, cfg.batch, cfg.n_prefix), dtype=torch.uint8,
                             device="cuda")

    def step():
        kv = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage)
        vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out=out)
        kv.close()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done at {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # ---- timed region: K whole steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    value = cfg.batch * args.steps / elapsed

    # ---- per-phase latency (separate, synchronised calls)
    pre_ms, den_ms, stp_ms = [], [], []
    for _ in range(5):
        kv, tp = vla.vla_prefix_encode(model, zt, kv_storage=kv_storage, timing=True)
        _, td = vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out=out, timing=True)
        kv.close()
        pre_ms.append(tp["prefix_ms"])
        den_ms.append(td["denoise_ms"])
        stp_ms.append(td["step_ms"])
    phases = {"prefix_ms": float(np.median(pre_ms)), "denoise_ms": float(np.median(den_ms)),
              "denoise_step_ms": float(np.median(stp_ms))}
    pf = prefix_flops(cfg) * cfg.batch
    absorbed = absorbed_form(vla, model, cfg)
    sb = expert_step_bytes(cfg, absorbed)
    prefix_peak = PEAK_INT8_TOPS if cfg.precision == "w2a8" else PEAK_BF16_TFLOPS
    phases["prefix_mfma_frac"] = pf / (phases["prefix_ms"] * 1e-3) / (prefix_peak * 1e12)
    phases["denoise_hbm_frac"] = sb / (phases["denoise_step_ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9)
    phases["denoise_mfma_frac"] = expert_step_flops(cfg) / (phases["denoise_step_ms"] * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)

    # ---- roofline of the kernel with the largest share of GPU time, and one entry per phase
    roofline = None if args.no_roofline else dominant_kernel_roofline(vla, model, cfg, zt, xt, out, kv_storage,
                                                                       absorbed)
    d_gbs = sb / (phases["denoise_step_ms"] * 1e-3) / 1e9
    p_rate = pf / (phases["prefix_ms"] * 1e-3) / 1e12
    roofline_phases = {
        "prefix": {"bound": "mfma", "achieved": p_rate, "peak": prefix_peak,
                   "unit": "TOP/s" if cfg.precision == "w2a8" else "TFLOP/s", "frac": p_rate / prefix_peak,
                   "work_per_pass": pf, "ms": phases["prefix_ms"]},
        "denoise": {"bound": "hbm", "achieved": d_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": d_gbs / PEAK_HBM_GBS,
                    "bytes_per_step": sb, "step_ms": phases["denoise_step_ms"],
                    "traffic": DENOISE_TRAFFIC_BYTES_PER_STEP if (args.config == 1 and args.attn == "cross" and absorbed)
                    else None},
    }

    # ---- solver-step sweep (Eq. 3) and the two-stream pipelined rate: context, not the metric
    extras = {}
    if args.config == 1 and args.attn == "cross" and not args.no_batched:
        extras["batched16"] = batched_entry(vla, model, cfg)
    if not args.no_extras:
        extras["solver_sweep"] = solver_sweep(vla, model, zt, xt, kv_storage)
        extras["w2a8_ablation"] = w2a8_ablation(vla)
    if args.pipelined:
        extras["pipelined_two_stream"] = pipelined(vla, model, cfg, zt, xt, max(args.steps, 10))

    # ---- CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w, betas, z0, x0, args.cpu_sample_s)

    model.close()
    rec = {
        "metric": "action chunks/s at batch 1 (prefix+denoise), % of MFMA / HBM roofline",
        "value": value, "unit": "chunks/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[cfg.precision], "data": "synthetic",
        "config": {"workload": cfg.name, "attention": cfg.attn, "batch": cfg.batch, "prefix_tokens": cfg.n_prefix,
                   "prefix_layers": cfg.L_p, "d_prefix": cfg.d_p, "expert_layers": cfg.L_e, "d_expert": cfg.d_e,
                   "chunk": [cfg.H, cfg.d_a], "solver_steps": cfg.steps},
        "phases": phases,
        "roofline": roofline,
        "roofline_phases": roofline_phases,
        "cpu_baseline": cpu,
        **extras,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(cfg, w, betas, z0, x0, budget_s):
    """The oracle, as it stands, on host cores: prefix layers then solver steps, stopped at the budget.

    Time per chunk is extrapolated from the measured per-layer costs: the prefix
    layers actually run, and whole expert velocity evaluations actually run.
    """
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    o = oracle.Oracle(cfg, w, betas)
    t0 = time.perf_counter()
    h = np.asarray(z0[0], dtype=np.float64)
    layers_done = 0
    kv = []
    for l in range(cfg.L_p):
        h, k, v = o.prefix_layer_kv(h, l)
        kv.append((k, v))
        layers_done += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    t_pre = (time.perf_counter() - t0) / layers_done * cfg.L_p
    t1 = time.perf_counter()
    if cfg.attn == "joint":  # the layers' own K/V (layers not run reuse the last ones: timing only)
        cache = [kv[min(l, len(kv) - 1)] for l in range(cfg.L_e)]
    else:
        cache = o.cache_project(oracle.rms_norm(h, o._w("prefix.norm"), cfg.rms_eps))
    t_cache = time.perf_counter() - t1
    x = np.asarray(x0[0], dtype=np.float64)
    sched = oracle.uniform_schedule(cfg.steps)
    t2 = time.perf_counter()
    steps_done = 0
    for k in range(cfg.steps):
        x = x + (sched[k + 1] - sched[k]) * o.velocity(x, sched[k], cache)
        steps_done += 1
        if time.perf_counter() - t2 > budget_s / 2:
            break
    t_step = (time.perf_counter() - t2) / steps_done
    t_chunk = t_pre + t_cache + cfg.steps * t_step
    return {"value": 1.0 / t_chunk, "unit": "chunks/s", "cores": threads, "kind": "oracle",
            "sample": f"one observation: {layers_done} of {cfg.L_p} prefix layers, "
                      f"{'the per-layer K/V' if cfg.attn == 'joint' else 'the cache projection'} and "
                      f"{steps_done} of {cfg.steps} solver steps run in float64 numpy, the rest extrapolated "
                      f"from the measured per-layer and per-step times",
            "seconds_measured": time.perf_counter() - t0,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
