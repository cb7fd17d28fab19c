"""Benchmark of the gated delta rule hot path on one MI355X.

A step is one gdn_chunk_fwd call over the prefill workload (B=4 sequences x T=4096 tokens, H=16
heads, d_k=d_v=128, bf16 q/k/v, fp32 gates, fp32 initial state ~N(0, 0.02), chunk 64): every
prefill row of the path runs inside it.  Inputs are resident in HBM before the timed region.
To keep the 256 MB Infinity Cache from serving the inputs, the timed loop rotates over several
independent copies of the inputs (more than twice the cache in total).

The JSON line reports prefill tokens/s as `value` (the K timed calls in groups of at least 10
consecutive calls between HIP events on the launch stream; the median over the groups of the mean
call time), the HBM roofline of the prefill kernel (algorithmic bytes per call / that time), the bf16
MFMA fraction under algorithmic flop accounting, the decode step (256 sequences x 32 heads, state
updated in place) as GB/s against HBM, the long-sequence prefill (1 x 262144 tokens, 16 heads,
segmented) and the packed variable-length prefill with the conv prologue (64 sequences of
512..16384 tokens, 32 heads) as tokens/s and GB/s, the prefill step with raw gate inputs and with
value heads sharing query/key heads and with the output epilogue, the decode step with the conv
prologue and a conv state (and with the fused epilogue as well), and the fp64 CPU oracle's
throughput on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
       python bench.py --record-traffic DIR   (no GPU: writes profiles/traffic.json from the
           rocprofv3 counter runs DIR/{fetch,write,cfetch,cwrite}/run_counter_collection.csv:
           FETCH_SIZE and WRITE_SIZE over `bench.py --steps 3 --warmup 1 --no-cpu-baseline
           --copies 1 --no-extra` and over `bench.py --copy-calibration`)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA, TFLOP/s
C_ACCOUNT = 64               # chunk length used for the algorithmic flop count


def prefill_alg_flops_per_token_head(dk, dv, C=C_ACCOUNT):
    """Triangles only: K K^T strict lower, Q K^T and Pm U lower incl. diagonal, forward
    substitution on [beta Gamma K | beta V], plus the three state products."""
    return 2 * (C * dk + (C - 1) * (dk + dv) / 2 + (C + 1) * dv / 2 + 3 * dk * dv)


def prefill_alg_bytes(tokens, N, H, dk, dv, with_states=True):
    per_th = (2 * dk + dv) * 2 + dv * 2 + 8   # q, k, v, o (bf16) + g, beta (fp32)
    b = tokens * H * per_th
    if with_states:
        b += 2 * N * H * dv * dk * 4
    return b


def decode_alg_bytes(N, H, dk, dv):
    return N * H * (2 * dv * dk * 4 + (2 * dk + dv) * 2 + dv * 2 + 8)


def load_traffic(kernel_tag):
    """HBM traffic per call measured with rocprofv3 counters (profiles/traffic.json), valid only
    while the hashes of the sources recorded with the counters still match."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_tag)
    except Exception:
        return None
    if not rec:
        return None
    shas = dict(rec.get("also", {}))
    shas[rec["source"]] = rec["source_sha"]
    for name, want in shas.items():
        if source_sha(name) != want:
            return None
    return rec["bytes_per_launch"]


def source_sha(name):
    import hashlib
    src = os.path.join(ROOT, "linear_attention_sequence_rule_amd", "csrc", name)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def _rerun_instantiation(name):
    """True for a chunk_bf16_kernel name whose LEAN template argument (the fifth) is false."""
    args = name.split("chunk_bf16_kernel<", 1)[1].split(">", 1)[0].split(",")
    return args[4].strip() == "false"


def record_traffic(d, out_path=None):
    """profiles/traffic.json from four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, KiB per
    dispatch, over a short bench run and over the plain-copy calibration).  The copy calibration
    gives the scale of each counter: bytes the copy moves each way / what the counter reads.  A
    prefill call is its chunk_bf16 dispatches: the main pass, then the transition and rerun passes
    in one launch (chunk_bf16_tail_kernel, counted once per call); where those two run as launches
    of their own, the rerun pass, the one instantiation with the rerun code, is counted instead."""
    import csv
    from collections import defaultdict

    def load(sub):
        per = defaultdict(list)
        for r in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            per[(int(r["Dispatch_Id"]), r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return {k: sum(v) for k, v in per.items()}  # one value per dispatch (summed over dimensions)

    scale = {}
    for sub, ctr in (("cfetch", "FETCH_SIZE"), ("cwrite", "WRITE_SIZE")):
        vals = [v for (_, name), v in load(sub).items() if "copyBuffer" in name]
        assert vals, "no copy kernel in " + sub
        scale[ctr] = (1 << 30) / (sum(vals) / len(vals) * 1024.0)
    out = {}
    fetch, write = load("fetch"), load("write")
    for tag, src, also in (("chunk_bf16_kernel", "chunk_bf16.hip", ("segments.hip", "api.hip")),
                           ("step_kernel", "step.hip", ())):
        tags = (tag, "chunk_bf16_tail_kernel") if tag == "chunk_bf16_kernel" else (tag,)
        fb = sum(v for (_, n), v in fetch.items() if any(t in n for t in tags)) * 1024.0 * scale["FETCH_SIZE"]
        wb = sum(v for (_, n), v in write.items() if any(t in n for t in tags)) * 1024.0 * scale["WRITE_SIZE"]
        if tag == "chunk_bf16_kernel":
            calls_f = sum(1 for (_, n) in fetch if "chunk_bf16_tail_kernel" in n)
            calls_w = sum(1 for (_, n) in write if "chunk_bf16_tail_kernel" in n)
            per = "prefill step: main pass + transition and rerun passes (one launch)"
            if not calls_f:
                # separate transition and rerun launches: the rerun pass has the only
                # instantiation with rerun code, template argument LEAN (the fifth:
                # <DK, BV, RAW, EPI, LEAN, ...>) false
                calls_f = sum(1 for (_, n) in fetch if tag in n and _rerun_instantiation(n))
                calls_w = sum(1 for (_, n) in write if tag in n and _rerun_instantiation(n))
                per = "prefill step: main pass + transition pass + rerun pass"
        else:
            calls_f = sum(1 for (_, n) in fetch if tag in n)
            calls_w = sum(1 for (_, n) in write if tag in n)
            per = "decode step"
        assert calls_f and calls_w, tag
        out[tag] = {"source": src, "source_sha": source_sha(src), "also": {a: source_sha(a) for a in also},
                    "bytes_per_launch": fb / calls_f + wb / calls_w, "fetch_bytes": fb / calls_f,
                    "write_bytes": wb / calls_w, "calls": [calls_f, calls_w], "per": per,
                    "counter_scale": dict(scale)}
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl):
    """The fp64 oracle timed on this host's cores: the prefill workload on all cores (the headline
    baseline) and on one thread, and bounded samples of the long, decode and varlen workloads."""
    import numpy as np
    import oracle
    from linear_attention_sequence_rule_amd import workloads as W

    def fwd(w, nthreads=0, pairs=None):
        cu = np.concatenate([[0], np.cumsum(w.lengths)])
        t = time.perf_counter()
        _, _, used = oracle.forward(w.as_float("q"), w.as_float("k"), w.as_float("v"), w.g, w.beta, w.s0, cu,
                                    w.conv_w, nthreads=nthreads, pairs=pairs)
        return time.perf_counter() - t, int(used)

    tokens = wl.T_tot
    all_s, used = fwd(wl)
    # one thread: the first sequence's 16 heads (a quarter of the prefill workload's chains)
    one = [(0, h) for h in range(wl.H)]
    one_s, _ = fwd(wl, nthreads=1, pairs=one)
    one_tok = int(wl.lengths[0])  # the sequence's tokens, every head
    extra = {}
    # long prefill: all 16 heads (262144 tokens each), all cores
    lw = W.long_prefill()
    ls, lu = fwd(lw)
    extra["long_prefill"] = {"value": lw.T_tot / ls, "unit": "tokens/s", "cores": lu, "seconds": ls,
                             "sample": "the whole workload (1 x 262144 tokens, 16 heads)"}
    del lw
    # decode: the whole step (256 x 32 chains of one token), all cores and one thread
    dw = W.decode()
    t = time.perf_counter()
    oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state)
    ds = time.perf_counter() - t
    t = time.perf_counter()
    oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state, nthreads=1)
    d1 = time.perf_counter() - t
    dbytes = decode_alg_bytes(dw.N, dw.H, dw.dk, dw.dv)
    extra["decode"] = {"value": dbytes / ds / 1e9, "unit": "GB/s", "seconds": ds, "one_thread_seconds": d1,
                       "one_thread_value": dbytes / d1 / 1e9,
                       "sample": "the whole step (256 sequences x 32 heads, fp64 state copy included)"}
    del dw
    # varlen: the 16 shortest-index sequences (a quarter of the 64), every head, conv prologue
    vw = W.varlen()
    vs = list(range(16))
    vpairs = [(n, h) for n in vs for h in range(vw.H)]
    vsec, vu = fwd(vw, pairs=vpairs)
    vtok = int(np.sum(vw.lengths[vs]))
    extra["varlen"] = {"value": vtok / vsec, "unit": "tokens/s", "cores": vu, "seconds": vsec,
                       "sample": "sequences 0..15 of the 64 (%d tokens), all 32 heads, conv + SiLU" % vtok}
    del vw
    return {"value": tokens / all_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "the whole prefill workload (4 x 4096 tokens, 16 heads), fp64 token-by-token recurrence, "
                      "threads over (sequence, head) chains; %.2f s" % all_s,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread": {"value": one_tok / one_s, "unit": "tokens/s", "cores": 1, "seconds": one_s,
                           "sample": "sequence 0 of the prefill workload (4096 tokens x 16 heads) on one thread"},
            "workloads": extra}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-sequence and varlen lines")
    ap.add_argument("--lines", default=None,
                    help="comma-separated subset of the extra lines to run (long_prefill, varlen, prefill_raw_gates, "
                         "prefill_grouped_heads, prefill_epilogue, prefill_slow_decay, decode_conv: with decode_full); "
                         "default all")
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated through the timed loop")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic.json from the rocprofv3 counter runs under DIR (no GPU)")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs the gated delta rule on a single device "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import linear_attention_sequence_rule_amd as gdn
    from linear_attention_sequence_rule_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        # 1 GiB read + 1 GiB written per copy: the scale for FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": src.numel() * 4, "launches": 3}))
        return

    def to_dev(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def settle(fn):
        # untimed calls for at least 50 ms: the GPU idles while each workload is generated on the
        # host, and its clocks need that long to come back up
        t_w, n_w = time.perf_counter(), 0
        while n_w < 2 or time.perf_counter() - t_w < 0.05:
            fn()
            torch.cuda.synchronize()
            n_w += 1

    # ---------------------------------------------------------------- prefill (the step)
    wl = W.prefill()
    N, H, dk, dv, T = wl.N, wl.H, wl.dk, wl.dv, wl.T_tot // wl.N
    tokens = wl.T_tot
    base = [to_dev(x) for x in (wl.q, wl.k, wl.v, wl.g, wl.beta, wl.s0)]
    copies = [base] + [[t.clone() for t in base] for _ in range(args.copies - 1)]
    outs = [(torch.empty((tokens, H, dv), dtype=torch.bfloat16, device=dev),
             torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)) for _ in copies]
    # the segment workspace, allocated once as a caller would (the binding would otherwise
    # allocate one per call)
    ws = torch.empty(max(gdn.gdn_chunk_workspace_size(N, tokens, H, dk, dv), 16), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, g, b, s0 = copies[i % len(copies)]
        o, sf = outs[i % len(outs)]
        gdn.gdn_chunk_fwd(q, k, v, g, b, s0, N=N, o=o, final_state=sf, workspace=ws, stream=stream)

    # the K timed calls in groups of G consecutive calls, each group between two HIP events on the
    # launch stream; the step time is the median over the groups of the per-call mean.  A group
    # holds at least 10 calls: the two event commands around a group cost the stream some
    # microseconds, which a group of 2 calls of ~100 us would report as ~5% of the step.  The
    # events are recorded once before anything is timed: the first use of timing events in a
    # process has been seen to hold the host for tens of milliseconds, during which the GPU idles
    # and its clocks drop.
    G = max(1, min(args.steps, max(10, args.steps // 10)))
    groups = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range((args.steps + G - 1) // G)]
    for a, b in groups:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    # then calls back to back, as in the timed region, for at least 0.2 s whatever --warmup says:
    # the clocks settle to their level under this load only after tens of milliseconds of it
    n_settle, t_s = args.warmup, time.perf_counter()
    while time.perf_counter() - t_s < 0.2:
        for _ in range(20):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    n_settle = [n_settle]
    t0 = time.perf_counter()
    i = 0
    for a, b in groups:
        a.record(stream)
        for _ in range(min(G, args.steps - i)):
            step(n_settle[0] + i)
            i += 1
        b.record(stream)
    torch.cuda.synchronize()
    wall_per_step = (time.perf_counter() - t0) / args.steps
    per_call = sorted(a.elapsed_time(b) * 1e-3 / min(G, args.steps - G * j) for j, (a, b) in enumerate(groups))
    m = len(per_call)
    median_s = per_call[m // 2] if m % 2 else 0.5 * (per_call[m // 2 - 1] + per_call[m // 2])
    ms_per_step = median_s * 1e3

    alg_bytes = prefill_alg_bytes(tokens, N, H, dk, dv)
    alg_flops = tokens * H * prefill_alg_flops_per_token_head(dk, dv)
    gbs = alg_bytes / median_s / 1e9
    tflops = alg_flops / median_s / 1e12
    value = tokens / median_s

    # ---------------------------------------------------------------- decode
    dw = W.decode()
    dq, dk_, dv_, dg, db, st = (to_dev(x) for x in (dw.q, dw.k, dw.v, dw.g, dw.beta, dw.state))
    od = torch.empty_like(dv_)
    settle(lambda: gdn.gdn_recurrent_step(dq, dk_, dv_, dg, db, st, o=od, stream=stream))
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in dev_ev:
        a.record(stream)
        gdn.gdn_recurrent_step(dq, dk_, dv_, dg, db, st, o=od, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    dec_s = sum(a.elapsed_time(b) for a, b in dev_ev) / len(dev_ev) * 1e-3
    dec_bytes = decode_alg_bytes(dw.N, dw.H, dw.dk, dw.dv)
    dec_gbs = dec_bytes / dec_s / 1e9

    # ---------------------------------------------------------------- long sequence, varlen + conv
    def timed(fn, iters):
        settle(fn)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return ts[len(ts) // 2] * 1e-3

    extra = {}
    picked = None if args.lines is None else set(args.lines.split(","))

    def want(name):
        return picked is None or name in picked

    if not args.no_extra and want("long_prefill"):
        lw = W.long_prefill()
        lq, lk, lv, lg, lb = (to_dev(x) for x in (lw.q, lw.k, lw.v, lw.g, lw.beta))
        lo = torch.empty_like(lv)
        lsf = torch.empty((lw.N, lw.H, lw.dv, lw.dk), dtype=torch.float32, device=dev)
        need = gdn.gdn_chunk_workspace_size(lw.N, lw.T_tot, lw.H, lw.dk, lw.dv)
        lws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        ls = timed(lambda: gdn.gdn_chunk_fwd(lq, lk, lv, lg, lb, None, N=lw.N, o=lo, final_state=lsf, workspace=lws,
                                             stream=stream), 5)
        lbytes = lw.T_tot * lw.H * ((2 * lw.dk + lw.dv) * 2 + lw.dv * 2 + 8) + lw.N * lw.H * lw.dv * lw.dk * 4
        extra["long_prefill"] = {
            "workload": "long prefill B=1 T=262144 H=16 dk=dv=128 bf16, zero initial state, segmented",
            "value": lw.T_tot / ls, "unit": "tokens/s", "us": ls * 1e6, "workspace_bytes": need,
            "hbm_alg_gbs": lbytes / ls / 1e9, "hbm_frac": lbytes / ls / 1e9 / HBM_PEAK_GBS}
        del lq, lk, lv, lg, lb, lo, lsf, lws, lw
    if not args.no_extra and want("varlen"):
        vw = W.varlen()
        vq, vk, vv, vg, vb, vs0, vcu, vcw = (to_dev(x) for x in (vw.q, vw.k, vw.v, vw.g, vw.beta, vw.s0, vw.cu_seqlens,
                                                                  vw.conv_w))
        vo = torch.empty_like(vv)
        vsf = torch.empty_like(vs0)
        # workspace, if the call needs one (allocated outside the timed region; none here: with
        # dk = dv = 128 the conv runs inside the chunk kernel)
        vneed = gdn.gdn_chunk_workspace_size(vw.N, vw.T_tot, vw.H, vw.dk, vw.dv, has_cu_seqlens=True, has_conv=True)
        vws = torch.empty(max(vneed, 16), dtype=torch.uint8, device=dev)
        vsec = timed(lambda: gdn.gdn_chunk_fwd(vq, vk, vv, vg, vb, vs0, vcu, vcw, o=vo, final_state=vsf, workspace=vws,
                                               stream=stream), 3)
        vbytes = vw.T_tot * vw.H * ((2 * vw.dk + vw.dv) * 2 + vw.dv * 2 + 8) + 2 * vw.N * vw.H * vw.dv * vw.dk * 4
        extra["varlen"] = {
            "workload": "varlen 64 sequences, lengths U{512..16384} (%d tokens), H=32, dk=dv=128 bf16, conv(4)+SiLU, "
                        "initial states; %s" % (vw.T_tot, "the conv runs inside the chunk kernel" if vneed == 0 else
                                                "the conv runs as a streaming pass into a %.1f GB workspace" % (vneed / 1e9)),
            "value": vw.T_tot / vsec, "unit": "tokens/s", "us": vsec * 1e6,
            "hbm_alg_gbs": vbytes / vsec / 1e9, "hbm_frac": vbytes / vsec / 1e9 / HBM_PEAK_GBS}
        del vq, vk, vv, vg, vb, vs0, vcu, vcw, vo, vsf, vw, vws
        torch.cuda.empty_cache()

    if not args.no_extra and want("prefill_raw_gates"):
        # the prefill step again, the gates formed in the kernel from the raw a, b, A_log, dt_bias
        ra, rb, rgp = (to_dev(x) for x in W.raw_gate_inputs(wl.meta["seed"], wl.lengths, H))
        q, k, v, _, _, s0 = copies[0]
        o, sf = outs[0]
        rsec = timed(lambda: gdn.gdn_chunk_fwd(q, k, v, ra, rb, s0, N=N, o=o, final_state=sf, gate_params=rgp,
                                               workspace=ws, stream=stream), 20)
        extra["prefill_raw_gates"] = {
            "workload": "prefill B=4 T=4096 H=16 dk=dv=128 bf16, raw gate inputs a, b [T,H] fp32 + A_log, dt_bias [H]",
            "value": tokens / rsec, "unit": "tokens/s", "us": rsec * 1e6,
            "hbm_alg_gbs": alg_bytes / rsec / 1e9, "hbm_frac": alg_bytes / rsec / 1e9 / HBM_PEAK_GBS}
        del ra, rb, rgp

    if not args.no_extra and want("prefill_grouped_heads"):
        # the prefill step with 16 value heads sharing 8 query/key heads (pairs of value heads read
        # one query/key head): the q, k bytes per value head halve
        gw = W.prefill(Hk=8)
        gq, gk, gv, gg, gb, gs0 = (to_dev(x) for x in (gw.q, gw.k, gw.v, gw.g, gw.beta, gw.s0))
        go, gsf = torch.empty_like(gv), torch.empty_like(gs0)
        gsec = timed(lambda: gdn.gdn_chunk_fwd(gq, gk, gv, gg, gb, gs0, N=N, o=go, final_state=gsf, workspace=ws,
                                               stream=stream), 20)
        gbytes = tokens * (gw.Hk * 2 * dk * 2 + H * (dv * 2 * 2 + 8)) + 2 * N * H * dv * dk * 4
        extra["prefill_grouped_heads"] = {
            "workload": "prefill B=4 T=4096, 16 value heads sharing 8 query/key heads, dk=dv=128 bf16",
            "value": tokens / gsec, "unit": "tokens/s", "us": gsec * 1e6,
            "hbm_alg_gbs": gbytes / gsec / 1e9, "hbm_frac": gbytes / gsec / 1e9 / HBM_PEAK_GBS}
        del gq, gk, gv, gg, gb, gs0, go, gsf, gw

    if not args.no_extra and want("prefill_epilogue"):
        # the prefill step with the output epilogue (zero-centred RMSNorm over dv, sigmoid output
        # gate), applied by the chunk kernel to its fp32 o
        ez = to_dev(W.f32_to_bf16_bits(np.random.default_rng([1, 77]).standard_normal((tokens, H, dv),
                                                                                      dtype=np.float32)))
        ew = to_dev(np.random.default_rng([1, 78]).normal(0.0, 0.2, size=dv).astype(np.float32))
        q, k, v, g, b, s0 = copies[0]
        o, sf = outs[0]
        esec = timed(lambda: gdn.gdn_chunk_fwd(q, k, v, g, b, s0, N=N, o=o, final_state=sf, out_gate=ez,
                                               norm_weight=ew, workspace=ws, stream=stream), 20)
        ebytes = alg_bytes + tokens * H * dv * 2 + dv * 4
        extra["prefill_epilogue"] = {
            "workload": "prefill B=4 T=4096 H=16 dk=dv=128 bf16 + output epilogue (RMSNorm over dv, sigmoid gate z "
                        "bf16 [T,H,dv]); the epilogue runs inside the chunk kernel",
            "value": tokens / esec, "unit": "tokens/s", "us": esec * 1e6,
            "hbm_alg_gbs": ebytes / esec / 1e9, "hbm_frac": ebytes / esec / 1e9 / HBM_PEAK_GBS}
        del ez, ew

    if not args.no_extra and want("prefill_slow_decay"):
        # the prefill step with slow decay everywhere (g = -1e-3, beta as drawn): no segment transition
        # is negligible, so every pass of the segmented path covers whole segments -- its worst case
        sg = torch.full_like(copies[0][3], -1e-3)
        q, k, v, _, b, s0 = copies[0]
        o, sf = outs[0]
        ssec = timed(lambda: gdn.gdn_chunk_fwd(q, k, v, sg, b, s0, N=N, o=o, final_state=sf, workspace=ws,
                                               stream=stream), 20)
        extra["prefill_slow_decay"] = {
            "workload": "prefill B=4 T=4096 H=16 dk=dv=128 bf16 with g = -1e-3 for every token (full segment "
                        "transitions and reruns)",
            "value": tokens / ssec, "unit": "tokens/s", "us": ssec * 1e6,
            "hbm_alg_gbs": alg_bytes / ssec / 1e9, "hbm_frac": alg_bytes / ssec / 1e9 / HBM_PEAK_GBS}
        del sg

    if not args.no_extra and want("decode_conv"):
        # the decode step with the conv prologue on the raw token (history in a conv state updated in
        # place) and raw gates: the decode side of a layer whose prefill ran the conv
        cw, hist = W.conv_inputs(3, dw.N, dw.H, dw.dk, dw.dv, "bf16")
        dcw, dcs = to_dev(cw), to_dev(hist)
        da, dbr, dgp = (to_dev(x) for x in W.raw_gate_inputs(3, np.ones(dw.N, np.int64), dw.H))
        csec = timed(lambda: gdn.gdn_recurrent_step(dq, dk_, dv_, da, dbr, st, o=od, gate_params=dgp, conv_w=dcw,
                                                    conv_state=dcs, stream=stream), 20)
        cbytes = dec_bytes + dw.N * 2 * 3 * dw.H * (2 * dw.dk + dw.dv) * 2 + dw.H * (2 * dw.dk + dw.dv) * 16
        dz = to_dev(W.f32_to_bf16_bits(np.random.default_rng([3, 77]).standard_normal((dw.N, dw.H, dw.dv),
                                                                                      dtype=np.float32)))
        dwn = to_dev(np.random.default_rng([3, 78]).normal(0.0, 0.2, size=dw.dv).astype(np.float32))
        nsec = timed(lambda: gdn.gdn_recurrent_step(dq, dk_, dv_, da, dbr, st, o=od, gate_params=dgp, conv_w=dcw,
                                                    conv_state=dcs, out_gate=dz, norm_weight=dwn, stream=stream), 20)
        nbytes = cbytes + dw.N * dw.H * dw.dv * 2 + dw.dv * 4
        extra["decode_full"] = {
            "workload": "decode 256 sequences x 32 heads, dk=dv=128: raw bf16 token -> conv(4)+SiLU (conv state in "
                        "place), raw gates, fp32 state in place, output epilogue fused (RMSNorm, sigmoid gate)",
            "value": nbytes / nsec / 1e9, "unit": "GB/s", "us_per_step": nsec * 1e6,
            "hbm_frac": nbytes / nsec / 1e9 / HBM_PEAK_GBS}
        del dz, dwn
        extra["decode_conv"] = {
            "workload": "decode 256 sequences x 32 heads, dk=dv=128, raw bf16 token -> conv(4)+SiLU with a bf16 conv "
                        "state updated in place, raw gates, fp32 state in place",
            "value": cbytes / csec / 1e9, "unit": "GB/s", "us_per_step": csec * 1e6,
            "hbm_frac": cbytes / csec / 1e9 / HBM_PEAK_GBS}
        del dcw, dcs, da, dbr, dgp

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    out = {
        "metric": "GDN chunked-prefill tokens/s (+% bf16 MFMA peak); decode-step GB/s (+% HBM)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=4 T=4096 H=16 dk=dv=128 bf16 q/k/v, fp32 gates and state, chunk 64",
                   "global_batch": N, "seq_len": T, "heads": H, "dk": dk, "dv": dv},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic("chunk_bf16_kernel")},
        "mfma": {"achieved_tflops_alg": tflops, "peak": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS,
                 "flops_per_token_head": prefill_alg_flops_per_token_head(dk, dv)},
        "prefill_call_us": median_s * 1e6,
        "prefill_timing": "median over %d groups of %d consecutive calls (HIP events on the launch stream) of the "
                          "per-call mean; host wall clock %.1f us per call" % (len(groups), G, wall_per_step * 1e6),
        "decode": {"workload": "decode 256 sequences x 32 heads, dk=dv=128, bf16 tokens, fp32 state in place",
                   "value": dec_gbs, "unit": "GB/s", "us_per_step": dec_s * 1e6,
                   "tokens_per_s": dw.N / dec_s,
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_gbs / HBM_PEAK_GBS, "traffic": load_traffic("step_kernel")}},
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
