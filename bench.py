"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_8k|prefill_64k|prefill_1m|fp32_small]
                    [--decode-steps 1000] [--no-cpu-baseline] [--no-packed] [--copy-probe-mib M]

One step = one kda_chunk_fwd call over the named prefill workload (default: bf16, B=1, H=32,
T=8192, d=128, C=64, S0=0), inputs already resident in HBM. The decode regime is measured in
the same run: `--decode-steps` chained kda_decode_step calls over 256 sequences x 32 heads
(fp32 state, bf16 tokens, each step its own pre-generated tokens), and so is a packed batch of
12 variable-length sequences (8192 tokens per head, 32 heads) with state checkpoints every 512
tokens (kda_chunk_fwd_varlen). Times come from HIP events recorded on the stream the library
launches on.

Prints one JSON line. `value` is prefill tokens/s (B*T / seconds per call). `roofline` is the
prefill call (all of its kernels: intra-chunk records, state passes, segment scan) against HBM
bandwidth with algorithmic bytes; its `traffic` is the HBM bytes per call that rocprofv3 counters
measured on the same sources (profiles/), null when the sources changed since. `decode` carries
the decode figures and its own roofline; `cpu_baseline` is the fp64 oracle timed on this host.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector/matrix, published

# Algorithmic work per token-head of chunkwise prefill (C = 64, dk = dv = d):
#   flops  6*dk*dv + C*(3*dk + 2*dv) + C^2/3      (state products, Gram/UT/causal halves)
#   bytes  q,k,log_alpha,v (4*d elements in) + beta (1) + o (d elements out)
# plus one fp32 state read (S0, when given) and one fp32 state write (S_T) per head.
def prefill_alg(B, H, T, d, in_bytes, out_bytes, has_s0, C=64):
    flops_tok = 6 * d * d + C * (5 * d) + C * C / 3.0
    bytes_tok = 4 * d * in_bytes + in_bytes + d * out_bytes
    state = d * d * 4 * (2 if has_s0 else 1)
    return B * H * T * flops_tok, B * H * (T * bytes_tok + state)


# Decode per (sequence, head): fp32 state read + write, q,k,log_alpha,v in, beta, o out.
def decode_alg(N, H, d, in_bytes=2, out_bytes=2):
    flops = 7 * d * d
    bytes_ = 2 * d * d * 4 + 4 * d * in_bytes + in_bytes + d * out_bytes
    return N * H * flops, N * H * bytes_


# Measured HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated) comes from the committed
# profile summary; a figure is used only while the kernel sources it was taken on are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_8k_and_decode.md")
PREFILL_SOURCES = ["kda_intra.hip", "kda_inter.hip", "kda_scan.hip", "kda_record.h", "kda_mfma.h", "kda_device.h",
                   "kda_plan.h", "kda_plan.cpp"]
DECODE_SOURCES = ["kda_decode.hip", "kda_device.h"]


def sources_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_78_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kind, workload_name, files):
    """Bytes per call/step recorded in the profile summary for this workload, or None."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    pat = r"traffic_bytes_per_%s\[(.*?)\] = (\d+) sources=([0-9a-f]+)" % kind
    for name, value, src in re.findall(pat, text):
        if name == workload_name and src == sources_hash(files):
            return int(value)
    return None


WORKLOADS = {
    "prefill_8k": "PREFILL_BF16_8K",
    "prefill_64k": "PREFILL_BF16_PREFIX_64K",
    "prefill_1m": "PREFILL_BF16_1M",
    "fp32_small": "PREFILL_FP32_SMALL",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_8k", choices=sorted(WORKLOADS))
    ap.add_argument("--segments", type=int, default=0, help="0 = the library's plan")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-packed", action="store_true", help="skip the packed variable-length batch")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward of the prefill workload")
    ap.add_argument("--cpu-lanes", type=int, default=32, help="lanes of the CPU-baseline sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    w = getattr(synth, WORKLOADS[args.workload])
    print("bench: generating %s" % w.name, file=sys.stderr, flush=True)
    q, k, v, la, beta, S0 = synth.workload_inputs(w, device=dev)
    out_dtype = w.dtype
    o = torch.empty(w.B, w.H, w.T, w.d, device=dev, dtype=out_dtype)
    S_T = torch.empty(w.B, w.H, w.d, w.d, device=dev, dtype=torch.float32)
    nbytes = kda.chunk_workspace_bytes(q, v, segments=args.segments)
    ws = torch.empty(max(nbytes, 16), device=dev, dtype=torch.uint8)

    def step():
        kda.chunk_fwd(q, k, v, la, beta, S0, out_dtype=out_dtype, segments=args.segments, o=o, S_T=S_T,
                      workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    call_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))
    tokens = w.B * w.T
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    flops, abytes = prefill_alg(w.B, w.H, w.T, w.d, in_b, in_b, S0 is not None)
    achieved_gbs = abytes / (call_ms * 1e-3) / 1e9
    tflops = flops / (call_ms * 1e-3) / 1e12
    mm_peak = BF16_PEAK_TFLOPS if w.dtype == torch.bfloat16 else FP32_PEAK_TFLOPS

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- packed variable-length batch with checkpoints ----------------
    packed = None
    if not args.no_packed:
        pw = synth.PACKED_BF16_8K
        lens = synth.PACKED_BF16_8K_LENS
        E = 512
        print("bench: packed %s" % pw.name, file=sys.stderr, flush=True)
        pq, pk, pv, pla, pbeta, cu, _ = synth.packed_inputs(lens, pw.H, pw.d, pw.d, pw.dtype, device=dev)
        N = len(lens)
        n_ck = sum(n // E for n in lens)
        po = torch.empty_like(pv)
        pS = torch.empty(N, pw.H, pw.d, pw.d, device=dev, dtype=torch.float32)
        pck = torch.empty(pw.T // E, pw.H, pw.d, pw.d, device=dev, dtype=torch.float32)
        poff = torch.empty(N + 1, device=dev, dtype=torch.int32)
        pws = torch.empty(max(kda.varlen_workspace_bytes(N, pw.H, pw.T, max(lens), pw.d, pw.d, ckpt_every=E), 16),
                          device=dev, dtype=torch.uint8)

        def pstep():
            kda.chunk_fwd_varlen(pq, pk, pv, pla, pbeta, cu, None, max_len=max(lens), ckpt_every=E, o=po, S_T=pS,
                                 S_ckpt=pck, ckpt_offsets=poff, workspace=pws, stream=stream)

        for _ in range(args.warmup):
            pstep()
        torch.cuda.synchronize()
        p0 = torch.cuda.Event(enable_timing=True)
        p1 = torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for _ in range(args.steps):
            pstep()
        p1.record(stream)
        torch.cuda.synchronize()
        pms = p0.elapsed_time(p1) / args.steps
        _, pby = prefill_alg(1, pw.H, pw.T, pw.d, 2, 2, False)
        pby += (N - 1) * pw.H * pw.d * pw.d * 4 + n_ck * pw.H * pw.d * pw.d * 4   # S_T per lane, checkpoints
        pgbs = pby / (pms * 1e-3) / 1e9

        # the same call with the fused prologue (decay from z) and epilogue (gate, RMSNorm)
        gz, gA, ggate, gw = synth.gating_inputs((pw.H, pw.T), pw.H, pw.d, pw.d, pw.dtype, device=dev)

        def fstep():
            kda.chunk_fwd_varlen(pq, pk, pv, None, pbeta, cu, None, max_len=max(lens), ckpt_every=E, o=po, S_T=pS,
                                 S_ckpt=pck, ckpt_offsets=poff, workspace=pws, stream=stream, z=gz, A_log=gA,
                                 gate=ggate, norm_weight=gw)

        for _ in range(args.warmup):
            fstep()
        torch.cuda.synchronize()
        p0.record(stream)
        for _ in range(args.steps):
            fstep()
        p1.record(stream)
        torch.cuda.synchronize()
        fms = p0.elapsed_time(p1) / args.steps
        fby = pby + pw.H * pw.T * pw.d * 2          # the gate rows (z replaces log_alpha)
        fgbs = fby / (fms * 1e-3) / 1e9
        del gz, gA, ggate, gw
        packed = {"workload": pw.name, "lengths": list(lens), "metric": "KDA packed prefill tokens/s",
                  "value": pw.T / (pms * 1e-3), "unit": "tokens/s", "ms_per_step": pms, "ckpt_every": E,
                  "checkpoints_per_call": n_ck,
                  "roofline": {"bound": "hbm", "achieved": pgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": pgbs / HBM_PEAK_GBS, "traffic": None},
                  "alg_bytes_per_call": pby,
                  "fused_gating": {"what": "decay from z (g = -5 sigmoid(e^A z)) and y = sigmoid(gate) RMSNorm(o)",
                                   "value": pw.T / (fms * 1e-3), "unit": "tokens/s", "ms_per_step": fms,
                                   "roofline": {"bound": "hbm", "achieved": fgbs, "peak": HBM_PEAK_GBS,
                                                "unit": "GB/s", "frac": fgbs / HBM_PEAK_GBS, "traffic": None},
                                   "alg_bytes_per_call": fby}}
        del pq, pk, pv, pla, pbeta, po, pws

    # ---------------- backward (training) of the same prefill workload ----------------
    bwd = None
    if not args.no_backward and w.dtype == torch.bfloat16:
        print("bench: backward %s" % w.name, file=sys.stderr, flush=True)
        g = torch.Generator(device=dev)
        g.manual_seed(17)
        dO = torch.randn(w.B, w.H, w.T, w.d, generator=g, device=dev).to(out_dtype)
        dST = torch.randn(w.B, w.H, w.d, w.d, generator=g, device=dev) * 0.1
        bws = torch.empty(max(kda.chunk_bwd_workspace_bytes(q, v, args.segments, out_dtype), 16), device=dev,
                          dtype=torch.uint8)

        def bstep():
            kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST, segments=args.segments, workspace=bws, stream=stream)

        for _ in range(max(1, args.warmup)):
            bstep()
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        nb = max(1, args.steps // 4)
        b0.record(stream)
        for _ in range(nb):
            bstep()
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / nb
        # bytes: the forward's inputs, dO in, fp32 gradients of q, k, v, log_alpha, beta out, states
        bby = w.B * w.H * (w.T * (4 * w.d * in_b + in_b + w.d * in_b + 4 * w.d * 4 + 4) + 3 * w.d * w.d * 4)
        bgbs = bby / (bms * 1e-3) / 1e9
        bwd = {"workload": w.name + ", backward (forward recompute included)", "metric": "KDA backward tokens/s",
               "value": tokens / (bms * 1e-3), "unit": "tokens/s", "ms_per_step": bms, "steps": nb,
               "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": bgbs / HBM_PEAK_GBS, "traffic": None},
               "alg_bytes_per_call": bby, "workspace_bytes": int(bws.numel())}
        del dO, bws

    # ---------------- decode regime ----------------
    decode = None
    if args.decode_steps > 0:
        dw = synth.DECODE_BF16_256x32
        print("bench: decode %s" % dw.name, file=sys.stderr, flush=True)
        S = synth.decode_state(dw.N, dw.H, dw.d, dw.d, dw.s_std, device=dev)
        toks = [synth.decode_tokens(dw.N, dw.H, dw.d, dw.d, dw.dtype, device=dev, seed=4000 + i)
                for i in range(min(args.decode_steps, 1000))]
        od = torch.empty(dw.N, dw.H, dw.d, device=dev, dtype=dw.dtype)
        for i in range(max(args.warmup, 3)):   # untimed, like the prefill's warm-up calls
            kda.decode_step(*toks[i % len(toks)], S, o=od, stream=stream)
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(args.decode_steps):
            kda.decode_step(*toks[i % len(toks)], S, o=od, stream=stream)
        d1.record(stream)
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1) / args.decode_steps
        dfl, dby = decode_alg(dw.N, dw.H, dw.d)
        dgbs = dby / (dms * 1e-3) / 1e9
        decode = {"workload": dw.name, "metric": "KDA decode tokens/s", "value": dw.N / (dms * 1e-3),
                  "unit": "tokens/s", "steps": args.decode_steps, "ms_per_step": dms,
                  "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": dgbs / HBM_PEAK_GBS,
                               "traffic": measured_traffic("step", dw.name, DECODE_SOURCES)},
                  "alg_bytes_per_step": dby, "alg_flops_per_step": dfl}
        del toks

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import native
        L = min(args.cpu_lanes, w.B * w.H)
        print("bench: cpu baseline (oracle) on %d lanes x %d tokens" % (L, w.T), file=sys.stderr, flush=True)
        f = lambda x: x.reshape((-1,) + tuple(x.shape[2:]))[:L].float().cpu().numpy()
        a = [f(q), f(k), f(v), f(la), f(beta)]
        s0 = None if S0 is None else f(S0)
        threads = native.default_threads()
        # repeat the sample until about 10 s of CPU work has been timed (bounded: at most 200 runs)
        runs, t0 = 0, time.perf_counter()
        while True:
            native.kda_fwd(*a, s0, threads=threads)
            runs += 1
            if time.perf_counter() - t0 >= 10.0 or runs >= 200:
                break
        dt = (time.perf_counter() - t0) / runs
        whole_s = dt * (w.B * w.H) / L          # lanes are independent: scale the sample to the workload
        cpu = {"value": w.B * w.T / whole_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "%d of %d lanes x %d tokens (fp64 token loop), %d runs, %.3f s each"
                         % (L, w.B * w.H, w.T, runs, dt)}

    line = {
        "metric": "KDA prefill tokens/s", "value": tokens / (call_ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.d, "dv": w.d, "chunk": 64,
                   "s0": S0 is not None, "segments": args.segments or "auto", "workspace_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("call", w.name, PREFILL_SOURCES)},
        "mfma": {"alg_tflops": tflops, "peak_tflops": mm_peak, "frac": tflops / mm_peak},
        "alg_bytes_per_call": abytes, "alg_flops_per_call": flops, "call_ms": call_ms,
        "decode": decode, "packed": packed, "backward": bwd, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
