"""Benchmark: Gated DeltaNet layer prefill on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: one GDN layer with 16 key heads and 32 value heads of width 128, bf16 activations,
fp32 state, width-4 causal conv with state, commit grid 512, sub-chunks of 64 rows; one step
commits T = 8192 rows (conv, L2 norm, gates, WY/UT factors, the state chain, outputs and the
new conv window).  Inputs are seeded synthetic tensors resident in HBM before timing starts;
three input sets rotate.

Timing protocol (cold cache): before each timed call a 512 MiB scratch buffer is read, which
evicts the 256 MB Infinity Cache and leaves it holding clean lines (a write would leave 256 MB
of dirty lines that the timed call then pays to write back); two HIP events on the launch stream
bracket the call.  `value` is T over the median call duration of the K timed steps
(`ms_per_step` is that median).  Per-kernel durations come from K more cold calls with HIP
events recorded by the library around each of its kernels (events between the kernels add to
the call, so those calls are not the timed ones).  The same K calls back to back without the
flush give the warm rate, labelled as such.

Prints one JSON line with those rates, a roofline object for the dominant kernel (its share of
the layer's algorithmic bytes over its average duration in the timed steps) and for the whole
call, the other workloads (the one-head fp32 layer; the multi-turn replay with forks; the
24-layer long session with checkpoints and a divergence; 32 batched branches against one
prefill per branch), the rows beside the layer (`extras`: state capture/restore, a 370-row
fork, decode steps of 1 and 32 sessions, the standalone conv, the two projections and the
full-attention layer), and the float64 CPU oracle timed on bounded samples.

    --no-extras             skip the rows beside the layer (`--extras` is accepted and is the
                            default)
    --no-workloads          skip the one-head and session workloads
    --copy-calibration N    run a plain N-byte device copy after timing (for counter scaling)
"""
import argparse
import hashlib
import json
import os
import sys
import time
import traceback

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


def warm_clock(call, seconds=0.25):
    """Repeat `call` for about `seconds` of wall time (untimed), so that a compute-bound kernel
    is timed at the clock it settles to under load rather than while the clock is still
    ramping up from the lighter work before it."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def algorithmic_flops(T, Hk, Hv, d, C=64):
    """Flops of the chunked method per call: K K^T and Q K^T per key head (lower triangle),
    and per value head the products with the state, the triangular T R and M D, and the
    state update (dense attention is not counted)."""
    mac_k = C * d                                        # per token per key head
    mac_v = 3 * d * d + ((C - 1) / 2 + (C + 1) / 2) * d + C * C / 6
    return 2.0 * T * (Hk * mac_k + Hv * mac_v)


def cpu_baseline(seconds_target=10.0):
    """The float64 oracle on bounded samples of the workloads: whole 8192-row calls of the
    16/32/128 layer (all 32 value heads, threads over heads) until about `seconds_target` of
    wall time; the same layer on one thread (1,024 rows); and the one-head fp32 layer (1,024
    rows, no conv).  The session workloads run the 16/32/128 layer shape, so their per-row
    oracle cost is the layer's."""
    import numpy as np
    from hybrid_linear_attention_prefill_amd import synth
    from oracle import c_oracle
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = nproc
    # the machine's CPU share for one GPU is 16 threads; the layer has 32 independent chains
    threads = max(1, min(16, avail, 32))
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
    n1 = 1024
    t0 = time.perf_counter()
    c_oracle.gdn_layer(x[:n1], w, np.zeros((3, shape.channels)), g[:n1], beta[:n1],
                       np.zeros((32, 128, 128)), threads=1, **kw)
    one = n1 / (time.perf_counter() - t0)
    c1 = synth.layer_inputs(synth.ONE_HEAD, 1024, seed=0, act_dtype=__import__("torch").float32,
                            unit_qk=True)
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 1.0:
        c_oracle.gdn_layer(synth.f64(c1["x"]), None, None, synth.f64(c1["g"]), synth.f64(c1["beta"]),
                           np.zeros((1, 64, 64)), n_k_heads=1, n_v_heads=1, d_k=64, d_v=64,
                           scale=64 ** -0.5, l2_eps=1e-6, threads=1)
        reps += 1
    c1_rate = reps * 1024 / (time.perf_counter() - t0)
    return {"value": calls * T_ROWS / spent, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "nproc": nproc, "cpus_available": avail,
            "one_thread_tokens_per_s": round(one, 1),
            "one_head_fp32_tokens_per_s": round(c1_rate, 1),
            "sample": "float64 per-token oracle (conv, L2 norm, gated delta rule) on the same "
                      "16/32/128 layer: %d whole 8192-row calls, %.1f s wall, %d threads over "
                      "heads; one thread on 1,024 rows; the one-head fp32 layer of 1,024 rows on "
                      "one thread" % (calls, spent, threads)}


def session_workloads(b, synth, desc, dev, shape):
    """Timed session-shaped workloads on the 16/32/128 layer (device time, inputs gathered
    on the device beforehand and outside the timed regions): a multi-turn replay with forks,
    a 24-layer long session with checkpoints, a divergence and re-prefill, and 32 batched
    branches against one prefill per branch."""
    import numpy as np
    import torch
    Hv, d = desc.n_v_heads, desc.d_v
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=2):
        fn()  # warm-up
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1e-3  # seconds per run

    def dev_rows(tab, ids):
        i = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=dev)
        return {"x": tab["E"][i], "g": tab["g"][i], "beta": tab["beta"][i]}

    def dev_table(vocab, seed):
        t = synth.TokenTables(shape, vocab, seed)
        return {"E": t.E.to(dev), "g": t.g.to(dev), "beta": t.beta.to(dev), "conv_w": t.conv_w.to(dev)}

    res = {}
    # 1. multi-turn replay: 41,802 tokens in 12 turns; after each turn the whole 512-row chunks
    #    are committed and the pending tail plus a 40-token question is forked
    total, n_turns, n_q, vocab, seed = 41802, 12, 40, 4096, 50
    tab = dev_table(vocab, seed)
    ids = synth.token_ids(seed, total, vocab)
    cuts = synth.turn_cuts(seed, total, n_turns)
    plan, committed = [], 0
    for t, end in enumerate(cuts):
        n = ((end - committed) // 512) * 512 if committed % 512 == 0 else 0
        fork_ids = np.concatenate([ids[committed + n:end], synth.question_ids(seed, t, n_q, vocab)])
        plan.append((dev_rows(tab, ids[committed:end]), end - committed, dev_rows(tab, fork_ids)))
        committed += n
    ws = b.workspace(desc, total)
    live, fork = b.State(desc), b.State(desc)
    o = torch.empty((total + n_q, Hv, d), dtype=torch.bfloat16, device=dev)

    def replay():
        b.gdn_state_init(desc, live)
        for rows, n, fk in plan:
            b.gdn_prefill_chunked(desc, rows["x"], tab["conv_w"], rows["g"], rows["beta"], live, live,
                                  o, n, b.GDN_COMMIT, ws)
            m = fk["x"].shape[0]
            b.gdn_prefill_chunked(desc, fk["x"], tab["conv_w"], fk["g"], fk["beta"], live, fork, o, m,
                                  b.GDN_FORK, ws)
    sec = timed(replay)
    fork_rows = sum(fk["x"].shape[0] for _, _, fk in plan)
    res["multi_turn_replay_41802"] = {
        "turns": n_turns, "committed_rows": committed, "fork_rows": int(fork_rows),
        "ms": round(sec * 1e3, 3), "session_tokens_per_s": round(total / sec, 1),
        "executed_rows_per_s": round((committed + fork_rows) / sec, 1)}
    del plan, tab, o

    # 2. long session: 24 layers, 100,000 tokens in 6 turns, a checkpoint of every layer at
    #    each turn end; then a divergence, a restore of the newest checkpoint at or below it
    #    and a re-prefill of the rest
    n_layers, total, n_turns, vocab, seed = 24, 100_000, 6, 1024, 60
    tabs = [dev_table(vocab, 1000 + l) for l in range(n_layers)]
    ids = synth.token_ids(seed, total, vocab)
    cuts = synth.turn_cuts(seed, total, n_turns)
    turns, committed = [], 0
    for end in cuts:
        n = ((end - committed) // 512) * 512
        turns.append((committed, n))
        committed += n
    inputs = [dev_rows(tabs[l], ids[:committed]) for l in range(n_layers)]
    d_pt = synth.divergence_point(seed, 1, total)
    ckpt_pos = [c + n for c, n in turns]
    k = max(i for i, p in enumerate([0] + ckpt_pos) if p <= d_pt) - 1
    p0 = ckpt_pos[k] if k >= 0 else 0
    ids2 = ids.copy()
    ids2[d_pt:] = synth.token_ids(seed + 1, total - d_pt, vocab)
    re_rows = ((total - p0) // 512) * 512
    inputs2 = [dev_rows(tabs[l], ids2[p0:p0 + re_rows]) for l in range(n_layers)]
    ws = b.workspace(desc, total)
    o = torch.empty((total, Hv, d), dtype=torch.bfloat16, device=dev)
    live = [b.State(desc) for _ in range(n_layers)]
    slots = [[b.State(desc) for _ in range(n_turns)] for _ in range(n_layers)]

    def session():
        for l in range(n_layers):
            b.gdn_state_init(desc, live[l])
        for t, (c0, n) in enumerate(turns):
            for l in range(n_layers):
                x = inputs[l]
                b.gdn_prefill_chunked(desc, x["x"][c0:c0 + n], tabs[l]["conv_w"], x["g"][c0:c0 + n],
                                      x["beta"][c0:c0 + n], live[l], live[l], o, n, b.GDN_COMMIT, ws)
                b.gdn_state_capture(desc, live[l], slots[l][t])

    def divergence():
        for l in range(n_layers):
            if k >= 0:
                b.gdn_state_restore(desc, live[l], slots[l][k])
            else:
                b.gdn_state_init(desc, live[l])
            x = inputs2[l]
            b.gdn_prefill_chunked(desc, x["x"], tabs[l]["conv_w"], x["g"], x["beta"], live[l], live[l],
                                  o, re_rows, b.GDN_COMMIT, ws)
    sec = timed(session, reps=1)
    sec2 = timed(lambda: (session(), divergence()), reps=1) - sec
    res["long_session_24_layers_100000"] = {
        "layers": n_layers, "committed_rows": committed, "turns": n_turns,
        "ms": round(sec * 1e3, 2), "tokens_per_s_per_layer": round(n_layers * committed / sec, 1),
        "divergence_at": int(d_pt), "restored_pos": int(p0), "reprefill_rows": int(re_rows),
        "restore_and_reprefill_ms": round(sec2 * 1e3, 2)}
    del inputs, inputs2, tabs, o, live, slots

    # 3. prefix sharing: request prefix 1,000, groups with 0/1/70/128 rows of their own, 8
    #    branches of 1-200 rows per group; prefixes run once up to their last multiple of 64,
    #    the branches in one batched call from the three shared states; against one plain
    #    prefill per branch of its whole prompt
    P, groups, per_group = 1000, [0, 1, 70, 128], 8
    lens = synth.branch_lengths(31 + P, len(groups) * per_group)
    tot = P + sum(groups) + sum(lens)
    dinp = {kk: v.to(dev) for kk, v in synth.layer_inputs(shape, tot, seed=31 + P).items()}

    def sub(idx):
        i = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=dev)
        return {kk: v[i] for kk, v in dinp.items() if kk != "conv_w"}
    gofs, bofs, cur, j = [], [], P, 0
    for gl in groups:
        gofs.append((cur, cur + gl))
        cur += gl
    for gi in range(len(groups)):
        for _ in range(per_group):
            bofs.append((gi, cur, cur + lens[j]))
            cur += lens[j]
            j += 1
    run_req = b.gdn_shared_prefix_rows(0, P)
    req_in = sub(range(run_req))
    g_plan = []
    for (g0, g1) in gofs:
        idx = list(range(run_req, P)) + list(range(g0, g1))
        run = b.gdn_shared_prefix_rows(run_req, run_req + len(idx))
        g_plan.append((sub(idx[:run]) if run else None, run, idx[run:]))
    rows, cu = [], [0]
    for (gi, b0, b1) in bofs:
        idx = g_plan[gi][2] + list(range(b0, b1))
        rows += idx
        cu.append(cu[-1] + len(idx))
    bx = sub(rows)
    fulls = [sub(list(range(0, P)) + list(range(*gofs[gi])) + list(range(b0, b1)))
             for (gi, b0, b1) in bofs]
    ws = b.workspace(desc, tot, 64)
    o = torch.empty((max(cu[-1], max(f["x"].shape[0] for f in fulls)), Hv, d), dtype=torch.bfloat16,
                    device=dev)
    zero, req, gst = b.State(desc), b.State(desc), [b.State(desc) for _ in groups]
    outs = [b.State(desc) for _ in bofs]
    b.gdn_state_init(desc, zero)
    cw = dinp["conv_w"]

    def shared():
        b.gdn_prefill_chunked(desc, req_in["x"], cw, req_in["g"], req_in["beta"], zero, req, o, run_req,
                              b.GDN_FORK, ws)
        inits = []
        for gi, (gin, run, _) in enumerate(g_plan):
            if run:
                b.gdn_prefill_chunked(desc, gin["x"], cw, gin["g"], gin["beta"], req, gst[gi], o, run,
                                      b.GDN_FORK, ws)
            inits.append(gst[gi] if run else req)
        b.gdn_prefill_branches(desc, cu, bx["x"], cw, bx["g"], bx["beta"],
                               [inits[gi] for (gi, _, _) in bofs], outs, o, ws)

    def per_branch():
        for k2, f in enumerate(fulls):
            b.gdn_prefill_chunked(desc, f["x"], cw, f["g"], f["beta"], zero, outs[k2], o, f["x"].shape[0],
                                  b.GDN_FORK, ws)
    full_rows = sum(f["x"].shape[0] for f in fulls)
    executed = run_req + sum(r for _, r, _ in g_plan) + cu[-1]
    s1, s2 = timed(shared, reps=5), timed(per_branch, reps=5)
    res["prefix_sharing_32_branches"] = {
        "request_prefix": P, "executed_rows": int(executed), "full_prompt_rows": int(full_rows),
        "shared_ms": round(s1 * 1e3, 3), "per_branch_ms": round(s2 * 1e3, 3),
        "shared_full_prompt_tokens_per_s": round(full_rows / s1, 1),
        "shared_executed_rows_per_s": round(executed / s1, 1),
        "per_branch_full_prompt_tokens_per_s": round(full_rows / s2, 1)}
    return res


def one_head_rate(b, synth, dev, reps=50):
    """The one-head fp32 layer (d = 64, T = 1,024, inputs post-conv, FORK from zero): tokens/s
    from the median of per-call HIP events.  Latency-bound (16 sub-chunks of one chain)."""
    import torch
    d1 = b.make_desc(1, 1, 64, 64, conv_width=0, act_dtype=torch.float32, out_dtype=torch.float32)
    inp = {k: v.to(dev) for k, v in synth.layer_inputs(synth.ONE_HEAD, 1024, seed=0,
                                                       act_dtype=torch.float32, unit_qk=True).items()}
    z, out = b.State(d1), b.State(d1)
    b.gdn_state_init(d1, z)
    o = torch.empty((1024, 1, 64), dtype=torch.float32, device=dev)
    ws = b.workspace(d1, 1024)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for _ in range(3):
        b.gdn_prefill_chunked(d1, inp["x"], None, inp["g"], inp["beta"], z, out, o, 1024, b.GDN_FORK, ws)
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        b.gdn_prefill_chunked(d1, inp["x"], None, inp["g"], inp["beta"], z, out, o, 1024, b.GDN_FORK, ws)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)[reps // 2]
    return {"T": 1024, "d": 64, "heads": 1, "dtype": "fp32", "us_median": round(ms * 1e3, 2),
            "tokens_per_s": round(1024 / (ms * 1e-3), 1)}


def measured_peaks(dev):
    """Reference rates measured on the box: a 1 GiB device-to-device copy (HBM read + write),
    and torch's bf16 matmul (the vendor BLAS) at the layer's two projection shapes, beside
    which the hand-written projection kernel is read."""
    import torch
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 10
    res = {"hbm_copy_GBps": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
           "hbm_copy_frac": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del src, dst
    for name, (T, K, N) in (("in_projection", (T_ROWS, 2048, 8256)), ("out_projection", (T_ROWS, 4096, 2048))):
        x = torch.randn((T, K), device=dev).to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev) / K ** 0.5).to(torch.bfloat16).t().contiguous()
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(x, w, out=y)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            torch.matmul(x, w, out=y)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        tf = 2.0 * T * K * N / (ms * 1e-3) / 1e12
        res["torch_matmul_" + name] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                                       "mfma_bf16_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        del x, w, y
    # torch's fused attention, restricted to its flash backend (no fallback to the unfused
    # path), at the full-attention layer's shape: 16 query heads over 2 key heads of width 256,
    # causal over 8,192 rows; key heads repeated to the query heads
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        import torch.nn.functional as F
        Hq, Hkv, D = 16, 2, 256
        q = torch.randn((1, Hq, T_ROWS, D), device=dev).to(torch.bfloat16)
        k = torch.randn((1, Hkv, T_ROWS, D), device=dev).to(torch.bfloat16)
        v = torch.randn((1, Hkv, T_ROWS, D), device=dev).to(torch.bfloat16)
        k = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(2):
                F.scaled_dot_product_attention(q, k, v, is_causal=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(5):
                F.scaled_dot_product_attention(q, k, v, is_causal=True)
            e1.record(stream)
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        tf = 4.0 * D * Hq * (T_ROWS * (T_ROWS + 1) / 2) / (ms * 1e-3) / 1e12
        res["torch_sdpa_flash_attention"] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                                             "mfma_bf16_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        del q, k, v
    except Exception as e:  # the flash backend may not support this shape or device
        res["torch_sdpa_flash_attention"] = {"unavailable": str(e)[:200]}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="time the rows beside the layer (the default): state capture/restore, "
                         "a 370-row fork, decode steps of 1 and 32 sessions, the standalone conv, "
                         "the two projections and the full-attention layer")
    ap.add_argument("--no-extras", action="store_true", help="skip the rows beside the layer")
    ap.add_argument("--peaks", action="store_true",
                    help="also measure a device copy and torch's bf16 matmul at the projection "
                         "shapes, as reference rates")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the one-head layer and the session workloads (multi-turn replay "
                         "with forks, the 24-layer long session, 32 batched branches)")
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
    stream = torch.cuda.current_stream()

    # Timed region: K steps, each a read of a 512 MiB scratch buffer (evicting the 256 MB
    # Infinity Cache, which then holds clean lines) and then one layer call, bracketed by two
    # HIP events on the launch stream, so that the call's duration excludes the flush.
    scratch = torch.ones((512 << 20) // 4, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int32, device=dev)
    names = ("prep_kernel", "chain_kernel")

    def fresh_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(args.steps)]
        for e in [e for row in evs for e in row]:
            e.record(stream)          # creates the underlying HIP events before timing
        return evs

    evs = fresh_events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        torch.amax(scratch, 0, out=sink)  # one reduction kernel that only reads the buffer
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = sorted(row[0].elapsed_time(row[1]) for row in evs)
    med_ms = call_ms[len(call_ms) // 2] if len(call_ms) % 2 else \
        0.5 * (call_ms[len(call_ms) // 2 - 1] + call_ms[len(call_ms) // 2])

    # Per-kernel durations: the same cold calls again, with HIP events recorded by the library
    # on the launch stream around each of its kernels (pair 0 the prep kernel, pair 1 the chain
    # kernel; pair 2 brackets no kernel).  Those events sit between the two kernels, so these
    # calls are not the ones timed above.
    kevs = fresh_events(6)
    torch.cuda.synchronize()
    for i in range(args.steps):
        torch.amax(scratch, 0, out=sink)
        step(i, kevs[i])
    torch.cuda.synchronize()
    per_kernel = {n: sum(row[2 * k].elapsed_time(row[2 * k + 1]) for row in kevs) / args.steps
                  for k, n in enumerate(names)}
    kernel_call_ms = sorted(row[0].elapsed_time(row[3]) for row in kevs)[args.steps // 2]
    del scratch, sink

    # Warm: the same K calls back to back (inputs and workspace partly in the Infinity Cache).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    tw = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - tw
    warm_ms = ev0.elapsed_time(ev1) / args.steps

    extras = {}
    # The rows beside the layer are reported, not the headline: a failure among them is
    # recorded in the line (and printed) instead of losing the layer's measurement.
    try:
        if not args.no_extras:
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
                # the same steps as a serving loop runs them: captured once in a HIP graph and
                # replayed, so that no host launch sits between two steps
                graph = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    with torch.cuda.graph(graph, stream=side):
                        for i in range(reps3):
                            src, dst = (ping, pong) if i % 2 == 0 else (pong, ping)
                            b.gdn_decode_step(desc, xb, s["conv_w"], gb, bb, src, dst, ob)
                torch.cuda.synchronize()
                graph.replay()
                e2.record(stream)
                graph.replay()
                e3.record(stream)
                torch.cuda.synchronize()
                graph_ms = e2.elapsed_time(e3) / reps3
                del graph
                step_bytes = B * (2 * Hv * d * d * 4 + 2 * 3 * C * 2 + C * 2 + 2 * Hv * 4 + Hv * d * 2)
                gbps = step_bytes / (step_ms * 1e-3) / 1e9
                ggbps = step_bytes / (graph_ms * 1e-3) / 1e9
                extras["decode_B%d" % B] = {
                    "us_per_step": round(step_ms * 1e3, 2),
                    "tokens_per_s": round(B / (step_ms * 1e-3), 1),
                    "algorithmic_bytes_per_step": step_bytes,
                    "achieved_GBps": round(gbps, 1),
                    "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
                    "us_per_step_graph": round(graph_ms * 1e3, 2),
                    "tokens_per_s_graph": round(B / (graph_ms * 1e-3), 1),
                    "hbm_frac_graph": round(ggbps / HBM_PEAK_GBS, 4)}
                del ping, pong

            # the standalone conv with its window over the layer's channels (bf16 in and out)
            cx = sets[0]["x"]
            cwin = torch.zeros((3, cx.shape[1]), dtype=torch.bfloat16, device=dev)
            cy = torch.empty_like(cx)
            warm_clock(lambda: b.conv1d_state_step(desc, cx, sets[0]["conv_w"], cwin, cy), 0.1)
            reps6 = 20
            e2.record(stream)
            for _ in range(reps6):
                b.conv1d_state_step(desc, cx, sets[0]["conv_w"], cwin, cy)
            e3.record(stream)
            torch.cuda.synchronize()
            conv_ms = e2.elapsed_time(e3) / reps6
            conv_bytes = 2 * cx.numel() * 2 + 4 * cx.shape[1] * 2 + 2 * 3 * cx.shape[1] * 2
            extras["conv1d_state_step"] = {"T": T_ROWS, "channels": int(cx.shape[1]),
                                           "us": round(conv_ms * 1e3, 2),
                                           "algorithmic_bytes": conv_bytes,
                                           "achieved_GBps": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                                           "hbm_frac": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del cwin, cy

            # the layer's projections at the prefill length (bf16 in and out, fp32 accumulation)
            for name, (K, N) in (("in_projection", (2048, 8256)), ("out_projection", (4096, 2048))):
                px = torch.randn((T_ROWS, K), device=dev).to(torch.bfloat16)
                pw = (torch.randn((N, K), device=dev) / K ** 0.5).to(torch.bfloat16)
                py = torch.empty((T_ROWS, N), dtype=torch.bfloat16, device=dev)
                warm_clock(lambda: b.gdn_linear(px, pw, py))
                reps4 = 50
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
            warm_clock(lambda: b.gdn_attention_prefill(adesc, [(aq, ak, av, ao, 0)]))
            reps5 = 20
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
    except Exception as e:  # noqa: BLE001
        traceback.print_exc()
        extras["error"] = repr(e)[:300]

    workloads = None
    if not args.no_workloads:
        try:
            workloads = {"one_head_fp32_T1024": one_head_rate(b, synth, dev)}
            workloads.update(session_workloads(b, synth, desc, dev, shape))
        except Exception as e:  # noqa: BLE001
            traceback.print_exc()
            workloads = {"error": repr(e)[:300]}
    if args.peaks:
        extras["measured_peaks"] = measured_peaks(dev)

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
    tokens_per_s = T_ROWS / (med_ms * 1e-3)
    dom = max(per_kernel, key=per_kernel.get)
    dom_achieved = split[dom] / (per_kernel[dom] * 1e-3) / 1e9
    layer_achieved = bytes_call / (med_ms * 1e-3) / 1e9
    ev_ms = med_ms
    out = {
        "metric": "Gated-DeltaNet prefill tokens/sec per layer (1 MI355X); % of MFMA/HBM roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 io, fp16 MFMA operands, fp32 accumulate and state",
        "data": "synthetic",
        "config": {"workload": "gdn_layer_commit_prefill", "T": T_ROWS, "n_k_heads": Hk,
                   "n_v_heads": Hv, "d_k": d, "d_v": d, "conv_width": 4, "grid": 512,
                   "sub_chunk": 64, "act_dtype": "bf16", "out_dtype": "bf16"},
        "timing": {
            "protocol": "cold cache: a 512 MiB scratch read before each timed call; value and "
                        "ms_per_step from the median of the per-call HIP event durations",
            "call_ms_median_with_kernel_events": round(kernel_call_ms, 5),
            "call_ms_median": round(med_ms, 5), "call_ms_min": round(call_ms[0], 5),
            "call_ms_max": round(call_ms[-1], 5),
            "call_ms_mean": round(sum(call_ms) / len(call_ms), 5),
            "timed_region_wall_s": round(wall, 4),
            "warm_back_to_back": {"tokens_per_s": round(T_ROWS * args.steps / warm_wall, 1),
                                  "ms_per_call_events": round(warm_ms, 5),
                                  "label": "warm: the K calls back to back, no flush"},
        },
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
    if workloads:
        out["workloads"] = workloads
    if extras:
        out["extras"] = extras
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
