"""Benchmark: Gated DeltaNet layer prefill on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: one GDN layer with 16 key heads and 32 value heads of width 128, bf16 activations,
fp32 state, width-4 causal conv with state, commit grid 512, sub-chunks of 64 rows; one step
commits T = 8192 rows (conv, L2 norm, gates, WY/UT factors, the state chain, outputs and the
new conv window).  Inputs are seeded synthetic tensors resident in HBM before timing starts;
three input sets rotate so that consecutive steps do not re-read the previous step's inputs
from the 256 MB Infinity Cache.

Prints one JSON line with the whole-job tokens/s (wall clock over the timed steps), a
roofline object for the dominant kernel (its share of the layer's algorithmic bytes over its
average duration, from HIP events the library records on the launch stream around each
kernel in every timed step), the same figure for the whole layer call, and the float64 CPU
oracle timed on a bounded sample of the same workload.

    --extras                also time state capture/restore, a 370-row fork, decode steps
                            of 1 and 32 sessions, the two projections and the attention layer
    --copy-calibration N    run a plain N-byte device copy after timing (for counter scaling)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense fp16 / bf16 MFMA
T_ROWS = 8192
SHAPE = dict(n_k_heads=16, n_v_heads=32, d=128)


def algorithmic_bytes(T, Hk, Hv, d, act_bytes=2, out_bytes=2):
    """HBM bytes the method must move per call: x (q|k|v) in, g and beta in, o out, the fp32
    state in and out, the conv window in and out, the conv weights in."""
    C = 2 * Hk * d + Hv * d
    per_token = C * act_bytes + 2 * Hv * 4 + Hv * d * out_bytes
    per_call = 2 * Hv * d * d * 4 + 2 * 3 * C * act_bytes + C * 4 * act_bytes
    return per_token, per_token * T + per_call


def kernel_bytes(T, Hk, Hv, d, act_bytes=2, out_bytes=2):
    """The same bytes split by the kernel that moves them between the caller's buffers and the
    chip: prep reads the q|k channels, g, beta and the conv weights; chain reads the v channels
    and the state, writes o and the state, and rewrites the conv window."""
    C = 2 * Hk * d + Hv * d
    prep = T * (2 * Hk * d * act_bytes + 2 * Hv * 4) + C * 4 * act_bytes
    chain = T * (Hv * d * act_bytes + Hv * d * out_bytes) + 2 * Hv * d * d * 4 + 2 * 3 * C * act_bytes
    return {"prep_kernel": prep, "chain_kernel": chain}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE and WRITE_SIZE counter runs stored
    in profiles/hbm_traffic_gdn_layer_T8192.txt, scaled by a plain copy's reading.  None when
    the file is missing or was taken from different kernel source than the one built now."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_gdn_layer_T8192.txt")
    src = os.path.join(ROOT, "hybrid_linear_attention_prefill_amd", "csrc", "gdn_kernels.hip")
    try:
        with open(path) as f:
            lines = f.read().splitlines()
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    fields = dict(ln.split("=", 1) for ln in lines if "=" in ln and not ln.startswith("#"))
    if fields.get("kernel_source_sha256") != digest:
        return None
    v = fields.get("bytes_per_launch." + kernel)
    return None if v is None else int(float(v))


def algorithmic_flops(T, Hk, Hv, d, C=64):
    """Flops of the chunked method per call: K K^T and Q K^T per key head (lower triangle),
    and per value head the products with the state, the triangular T R and M D, and the
    state update (dense attention is not counted)."""
    mac_k = C * d                                        # per token per key head
    mac_v = 3 * d * d + ((C - 1) / 2 + (C + 1) / 2) * d + C * C / 6
    return 2.0 * T * (Hk * mac_k + Hv * mac_v)


def cpu_baseline(seconds_target=10.0):
    """The float64 oracle on a bounded sample of the workload: whole 8192-row layer calls (all
    32 value heads, threads over heads), repeated until about `seconds_target` of wall time."""
    import numpy as np
    from hybrid_linear_attention_prefill_amd import synth
    from oracle import c_oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    shape = synth.LAYER_16x32x128
    kw = dict(n_k_heads=16, n_v_heads=32, d_k=128, d_v=128, scale=128 ** -0.5, l2_eps=1e-6)
    inp = synth.layer_inputs(shape, T_ROWS, seed=0)
    x, w = synth.f64(inp["x"]), synth.f64(inp["conv_w"])
    g, beta = synth.f64(inp["g"]), synth.f64(inp["beta"])
    calls, spent = 0, 0.0
    while spent < seconds_target:
        t0 = time.perf_counter()
        c_oracle.gdn_layer(x, w, np.zeros((3, shape.channels)), g, beta,
                           np.zeros((32, 128, 128)), threads=threads, **kw)
        spent += time.perf_counter() - t0
        calls += 1
    return {"value": calls * T_ROWS / spent, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "float64 per-token oracle (conv, L2 norm, gated delta rule) on the same "
                      "16/32/128 layer: %d whole 8192-row calls, %.1f s wall" % (calls, spent)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="also time state capture/restore, a 370-row fork, decode "
                         "steps of 1 and 32 sessions, the two projections and the full-attention "
                         "layer")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed region, run a plain device copy of BYTES bytes three "
                         "times (reference dispatch for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the layer's heads would shard across GPUs with no "
              "exchange step, but that path is not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_linear_attention_prefill_amd import binding as b
    from hybrid_linear_attention_prefill_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Hk, Hv, d = SHAPE["n_k_heads"], SHAPE["n_v_heads"], SHAPE["d"]
    desc = b.make_desc(Hk, Hv, d, d, conv_width=4, grid=512)
    shape = synth.LAYER_16x32x128

    n_sets = 3
    sets = []
    for i in range(n_sets):
        inp = synth.layer_inputs(shape, T_ROWS, seed=i)
        sets.append({k: v.to(dev) for k, v in inp.items()})
    o = torch.empty((T_ROWS, Hv, d), dtype=torch.bfloat16, device=dev)
    ws = b.workspace(desc, T_ROWS, 1)
    state = b.State(desc)
    b.gdn_state_init(desc, state)

    def step(i, events=()):
        s = sets[i % n_sets]
        n = b.gdn_prefill_chunked_events(desc, s["x"], s["conv_w"], s["g"], s["beta"], state,
                                         state, o, T_ROWS, b.GDN_COMMIT, ws, events=events)
        assert n == T_ROWS

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: K layer calls back to back (the throughput figure).
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    # Timed region 2: the same K calls with HIP events recorded by the library on the launch
    # stream around each of its three kernels (the per-kernel durations).
    # (the library's third event pair brackets no kernel: the chain kernel writes the window)
    names = ("prep_kernel", "chain_kernel")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e in [e for row in evs for e in row]:
        e.record(stream)              # creates the underlying HIP events before timing
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per_kernel = {n: sum(row[2 * k].elapsed_time(row[2 * k + 1]) for row in evs) / args.steps
                  for k, n in enumerate(names)}

    extras = {}
    if args.extras:
        # state copies (capture + restore of the 2 MiB state and window) and a fork of a
        # 330-row pending tail plus a 40-row question above the committed rows
        snap = b.State(desc)
        fork_out = b.State(desc)
        fo = torch.empty((370, Hv, d), dtype=torch.bfloat16, device=dev)
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps2 = 20
        e2.record(stream)
        for _ in range(reps2):
            b.gdn_state_capture(desc, state, snap)
            b.gdn_state_restore(desc, state, snap)
        e3.record(stream)
        torch.cuda.synchronize()
        copy_ms = e2.elapsed_time(e3) / reps2
        copy_bytes = 2 * 2 * (b.gdn_state_S_bytes(desc) + b.gdn_state_conv_bytes(desc))
        e2.record(stream)
        for _ in range(reps2):
            s = sets[0]
            b.gdn_prefill_chunked(desc, s["x"][:370], s["conv_w"], s["g"][:370], s["beta"][:370],
                                  state, fork_out, fo, 370, b.GDN_FORK, ws)
        e3.record(stream)
        torch.cuda.synchronize()
        extras = {"state_capture_restore_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
                  "fork_370_rows_ms": round(e2.elapsed_time(e3) / reps2, 4)}
        # decode steps of B sessions, each from its own forked state, in place: the step
        # streams every session's fp32 state in and out, so it is HBM-bound for large B
        C = desc.channels
        # (two states per session, stepped back and forth: one launch per step)
        for B in (1, 32):
            ping = [b.State(desc) for _ in range(B)]
            pong = [b.State(desc) for _ in range(B)]
            for st_ in ping:
                b.gdn_state_capture(desc, state, st_)
            s = sets[0]
            xb, gb, bb = s["x"][:B].contiguous(), s["g"][:B].contiguous(), s["beta"][:B].contiguous()
            ob = torch.empty((B, Hv, d), dtype=torch.bfloat16, device=dev)
            for i in range(4):
                src, dst = (ping, pong) if i % 2 == 0 else (pong, ping)
                b.gdn_decode_step(desc, xb, s["conv_w"], gb, bb, src, dst, ob)
            reps3 = 50
            e2.record(stream)
            for i in range(reps3):
                src, dst = (ping, pong) if i % 2 == 0 else (pong, ping)
                b.gdn_decode_step(desc, xb, s["conv_w"], gb, bb, src, dst, ob)
            e3.record(stream)
            torch.cuda.synchronize()
            step_ms = e2.elapsed_time(e3) / reps3
            step_bytes = B * (2 * Hv * d * d * 4 + 2 * 3 * C * 2 + C * 2 + 2 * Hv * 4 + Hv * d * 2)
            gbps = step_bytes / (step_ms * 1e-3) / 1e9
            extras["decode_B%d" % B] = {
                "us_per_step": round(step_ms * 1e3, 2),
                "tokens_per_s": round(B / (step_ms * 1e-3), 1),
                "algorithmic_bytes_per_step": step_bytes,
                "achieved_GBps": round(gbps, 1),
                "hbm_frac": round(gbps / HBM_PEAK_GBS, 4)}
            del ping, pong

        # the layer's projections at the prefill length (bf16 in and out, fp32 accumulation)
        for name, (K, N) in (("in_projection", (2048, 8256)), ("out_projection", (4096, 2048))):
            px = torch.randn((T_ROWS, K), device=dev).to(torch.bfloat16)
            pw = (torch.randn((N, K), device=dev) / K ** 0.5).to(torch.bfloat16)
            py = torch.empty((T_ROWS, N), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                b.gdn_linear(px, pw, py)
            reps4 = 20
            e2.record(stream)
            for _ in range(reps4):
                b.gdn_linear(px, pw, py)
            e3.record(stream)
            torch.cuda.synchronize()
            lin_ms = e2.elapsed_time(e3) / reps4
            tflops = 2.0 * T_ROWS * K * N / (lin_ms * 1e-3) / 1e12
            extras["linear_" + name] = {"T": T_ROWS, "K": K, "N": N,
                                        "us": round(lin_ms * 1e3, 2),
                                        "tflops": round(tflops, 1),
                                        "mfma_bf16_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}
            del px, pw, py

        # the hybrid's full-attention layer at the same length: 16 query heads over 2 key
        # heads of width 256, causal over 8,192 rows (flops: QK^T and PV over the causal
        # triangle, 4 D per query-key pair)
        Hq_a, Hkv_a, D_a = 16, 2, 256
        aq = torch.randn((T_ROWS, Hq_a, D_a), device=dev).to(torch.bfloat16)
        ak = torch.randn((T_ROWS, Hkv_a, D_a), device=dev).to(torch.bfloat16)
        av = torch.randn((T_ROWS, Hkv_a, D_a), device=dev).to(torch.bfloat16)
        ao = torch.empty_like(aq)
        adesc = b.make_attn_desc(Hq_a, Hkv_a, D_a)
        for _ in range(2):
            b.gdn_attention_prefill(adesc, [(aq, ak, av, ao, 0)])
        reps5 = 10
        e2.record(stream)
        for _ in range(reps5):
            b.gdn_attention_prefill(adesc, [(aq, ak, av, ao, 0)])
        e3.record(stream)
        torch.cuda.synchronize()
        att_ms = e2.elapsed_time(e3) / reps5
        att_flops = 4.0 * D_a * Hq_a * T_ROWS * (T_ROWS + 1) / 2
        att_tf = att_flops / (att_ms * 1e-3) / 1e12
        extras["attention_prefill"] = {"T": T_ROWS, "n_q_heads": Hq_a, "n_kv_heads": Hkv_a,
                                       "head_dim": D_a, "us": round(att_ms * 1e3, 1),
                                       "tflops": round(att_tf, 1),
                                       "mfma_bf16_frac": round(att_tf / MFMA_F16_PEAK_TFLOPS, 4)}
        del aq, ak, av, ao

    if args.copy_calibration:
        # a plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per_token, bytes_call = algorithmic_bytes(T_ROWS, Hk, Hv, d)
    split = kernel_bytes(T_ROWS, Hk, Hv, d)
    flops_call = algorithmic_flops(T_ROWS, Hk, Hv, d)
    tokens_per_s = T_ROWS * args.steps / wall
    dom = max(per_kernel, key=per_kernel.get)
    dom_achieved = split[dom] / (per_kernel[dom] * 1e-3) / 1e9
    layer_achieved = bytes_call / (ev_ms * 1e-3) / 1e9
    out = {
        "metric": "Gated-DeltaNet prefill tokens/sec per layer (1 MI355X); % of MFMA/HBM roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 io, fp16 MFMA operands, fp32 accumulate and state",
        "data": "synthetic",
        "config": {"workload": "gdn_layer_commit_prefill", "T": T_ROWS, "n_k_heads": Hk,
                   "n_v_heads": Hv, "d_k": d, "d_v": d, "conv_width": 4, "grid": 512,
                   "sub_chunk": 64, "act_dtype": "bf16", "out_dtype": "bf16"},
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(dom_achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom),
            "algorithmic_bytes_per_launch": split[dom],
            "launch_ms_events": round(per_kernel[dom], 5),
            "per_kernel_ms_events": {k: round(v, 5) for k, v in per_kernel.items()},
            "per_kernel_algorithmic_bytes": split,
            "layer_call": {
                "achieved": round(layer_achieved, 1),
                "frac": round(layer_achieved / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": bytes_call,
                "algorithmic_bytes_per_token": per_token,
                "call_ms_events": round(ev_ms, 5),
                "mfma_tflops_algorithmic": round(flops_call / (ev_ms * 1e-3) / 1e12, 2),
                "mfma_frac_algorithmic": round(flops_call / (ev_ms * 1e-3) / 1e12
                                               / MFMA_F16_PEAK_TFLOPS, 4),
            },
        },
    }
    if extras:
        out["extras"] = extras
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
