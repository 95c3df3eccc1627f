"""Benchmark: chunkwise retention forward at N=8192 (TFLOP/s, tokens/s) and the recurrent decode step
(GB/s) on one MI355X, printed as one JSON line.

One step = one chunkwise forward of the 6.7B-layer-shaped workload (B=1, H=16, N=8192, d_k=256,
d_v=512, chunk 128, bf16 inputs, fp32 accumulation, per-head GroupNorm eps 1e-5, bf16 output)
followed by one decode step of 128 sequences x 16 heads on fp32 256 x 512 states (made by a
chunkwise prefill of 8192 random bf16 tokens). Inputs are resident in HBM before timing starts.

Timing: W untimed warm-up steps, then K timed steps between device synchronisations; each part of
each step is bracketed with HIP events recorded on the stream the library launches on.

Counting rules:
  chunkwise algorithmic FLOPs per (b, h): 2 (d_k + d_v) * causal pairs inside chunks + 4 N d_k d_v
  decode algorithmic bytes: fp32 state read + write, bf16 q, k, v, fp32 out
  backward algorithmic FLOPs per (b, h): 2 (3 d_k + 2 d_v) * causal pairs + 10 N d_k d_v (the
    scores Q K^T and dout V^T, their products with K, Q and dout, and per token the five
    d_k x d_v products dout R^T, U v, U^T k and the two state updates)
  backward algorithmic bytes: bf16 q, k, v, dout read; fp32 dq, dk, dv written
  parallel form algorithmic FLOPs per (b, h): 2 (d_k + d_v) N (N + 1) / 2 (every causal pair)

Beside the step, outside its timed region: the same chunkwise call with a swish gate after the
GroupNorm, the parallel form of the same layer, the chunkwise call and the decode step with the
positional rotation of q and k, residual
linear attention at the same shape (512-token window, softmax feature map; its rate is counted with
the chunkwise FLOPs), and the chunkwise backward (dq, dk, dv) of the same workload with a bf16 dout,
each timed over the same K calls.

Also reported: the median and minimum per-call times of the step's two parts; the chunkwise call
with a cold cache (512 MiB written before each call); the long-context workload (N=65536, chunk 64
to 512, fp32 out); this GPU's own peaks from hand-written probes (bf16 MFMA rate, HBM read and copy
rates; the roofline fractions stay against the published peaks); the host CPU model for the oracle.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "chunkwise retention fwd TFLOP/s & tokens/s at N=8192; decode-step GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def chunk_flops(B, H, N, dk, dv, C):
    pairs = 0
    for c0 in range(0, N, C):
        L = min(C, N - c0)
        pairs += L * (L + 1) // 2
    return B * H * (2 * (dk + dv) * pairs + 4 * N * dk * dv)


def backward_flops(B, H, N, dk, dv, C):
    pairs = 0
    for c0 in range(0, N, C):
        L = min(C, N - c0)
        pairs += L * (L + 1) // 2
    return B * H * (2 * (3 * dk + 2 * dv) * pairs + 10 * N * dk * dv)


RLA_WINDOW = 512  # the window the RAttention page reports matching full attention with

# The only figures the pages print for this method are whole-model ones (abeam.tech RetNet summary,
# "Experiments": "Training cost" and "Inference cost"). Reported beside the kernel numbers as
# context only: another machine, a whole 6.7B model (every layer, projections, FFN, backward) in
# plain PyTorch, so neither a same-node nor a same-workload comparison, and no vs_baseline.
PAGES_CONTEXT = {
    "not_comparable": "whole 6.7B RetNet model on 8x A100 80GB in plain PyTorch without kernel fusion (training) and an "
                      "unstated setup (decoding); not this kernel, not this node",
    "training_words_per_s": 17458.6, "training_seq_len": 8192, "training_hardware": "8x A100 80GB",
    "training_memory_GB": 48.0,
    "decode_speedup_vs_kv_cache_transformer": 8.4, "decode_memory_saving_frac": 0.70, "decode_input_len": 8192,
    "source": "abeam.tech RetNet paper summary, Experiments: Training cost, Inference cost",
}


def time_calls(fn, n, stream, torch):
    """Average time of fn() over n calls, with HIP events on the library's stream."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3


def time_pair(base, variant, n, stream, torch):
    """Average times of base() and variant(), called alternately n times each with HIP events on the
    library's stream, so that clock drift over the run affects both alike."""
    base()
    variant()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for e in evs:
        e[0].record(stream)
        base()
        e[1].record(stream)
        variant()
        e[2].record(stream)
    torch.cuda.synchronize()
    tb = sum(e[0].elapsed_time(e[1]) for e in evs) / n * 1e-3
    tv = sum(e[1].elapsed_time(e[2]) for e in evs) / n * 1e-3
    return tb, tv


def chunk_bytes(B, H, N, dk, dv, in_bytes=2, out_bytes=2):
    return B * H * N * (2 * dk + dv) * in_bytes + B * H * N * dv * out_bytes


def decode_bytes(B, H, dk, dv):
    return B * H * (2 * dk * dv * 4 + (2 * dk + dv) * 2 + dv * 4)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_peaks(torch, dev, stream):
    """This GPU's own peaks from the hand-written probes (peak_probe.hip): dense bf16 MFMA rate
    (every wave issuing independent 32x32x16 MFMA chains, 8 waves per SIMD) and HBM rates (a 4 GiB
    read; a 1 GiB device copy, read + write). Each is the best of 3 timed launches. The roofline
    fractions stay against the published peaks; these say how much of them the chip reaches."""
    import ctypes
    path = os.path.join(ROOT, "libpeakprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nthr = lib.probe_threads()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best(fn, n=3):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * nthr, dtype=torch.float32, device=dev)
    t = best(lambda: lib.probe_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp))
    mfma_tflops = blocks * 4 * iters * 4 * 32768 / t / 1e12
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    rblocks = 256 * 16
    rout = torch.empty(rblocks * nthr, dtype=torch.float32, device=dev)
    t = best(lambda: lib.probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rblocks, ctypes.c_void_p(rout.data_ptr()), sp))
    read_gbps = nbytes / t / 1e9
    src, dst = buf[: (1 << 28)], torch.empty(1 << 28, dtype=torch.float32, device=dev)
    t = best(lambda: dst.copy_(src))
    copy_gbps = 2 * (1 << 30) / t / 1e9
    del buf, dst, out, rout
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "hbm_read_GBps": round(read_gbps, 1),
            "hbm_copy_GBps": round(copy_gbps, 1),
            "how": "peak_probe.hip: bf16 32x32x16 MFMA chains (2048 workgroups x 4 waves x 4096 trips x 4 MFMAs); "
                   "4 GiB non-temporal read; 1 GiB torch device copy counted as read + write; best of 3"}


def read_counters(name, kernel_sources):
    """HBM traffic per dispatch from a committed rocprofv3 counter summary, if it was taken on the
    current kernel source (sha256 recorded in the summary); else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    h = hashlib.sha256()
    for src in kernel_sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    try:
        return float(fields["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--peaks", action="store_true", help="only run the peak probes and print their JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (scale reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the retention path is "
              "single-GPU: heads and sequences are independent and would shard without communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_recurrent_sequence_chunkwise_amd import inputs as I
    from linear_recurrent_sequence_chunkwise_amd import retention as R

    R.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        n = 1 << 28  # fp32 elements: 1 GiB read and 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n, "copies": 3}))
        return

    if args.peaks:
        print(json.dumps(measured_peaks(torch, dev, stream)), flush=True)
        return

    # ---- chunkwise workload
    w = I.WORKLOADS["retention_b1_h16_n8192_dk256_dv512_bf16_gn"]
    C = w.chunks[0]
    q, k, v = (t.to(dev) for t in I.make_workload_qkv(w))
    gam = w.gamma_list()
    gn = R.GroupNorm(w.eps)
    out = torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.bfloat16, device=dev)
    st_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws_bytes = R.workspace_bytes(R.RET_FN_CHUNKWISE, w.B, w.H, w.N, w.dk, w.dv, torch.bfloat16, torch.bfloat16, C, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # ---- decode workload: state from a chunkwise prefill of 8192 tokens
    d = I.WORKLOADS["decode_b128_h16_dk256_dv512"]
    dgam = d.gamma_list()
    state = torch.empty((d.B, d.H, d.dk, d.dv), dtype=torch.float32, device=dev)
    per = 16
    for b0 in range(0, d.B, per):
        qp, kp, vp = I.make_qkv(per, d.H, I.DECODE_PREFILL_TOKENS, d.dk, d.dv, "bf16", seed=d.seed * 1000 + b0, device=dev)
        R.chunkwise_fwd(qp, kp, vp, dgam, 128, state_out=state[b0:b0 + per], want_out=False)
        del qp, kp, vp
    qn, kn, vn = (t[:, :, 0].contiguous().to(dev) for t in I.make_qkv(d.B, d.H, 1, d.dk, d.dv, "bf16", seed=d.seed))
    dout = torch.empty((d.B, d.H, d.dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("setup done")

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        R.chunkwise_fwd(q, k, v, gam, C, groupnorm=gn, out=out, state_out=st_out, workspace=ws, stream=stream)
        if evs:
            evs[1].record(stream)
        R.recurrent_step(qn, kn, vn, dgam, state, out=dout, stream=stream)
        if evs:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_chunk = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps * 1e-3
    t_dec = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e-3
    t_step = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps * 1e-3
    per_chunk = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in evs)
    per_dec = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in evs)
    timing = {"chunkwise_us": {"mean": round(t_chunk * 1e6, 2), "median": round(per_chunk[len(per_chunk) // 2], 2),
                               "min": round(per_chunk[0], 2)},
              "decode_us": {"mean": round(t_dec * 1e6, 2), "median": round(per_dec[len(per_dec) // 2], 2),
                            "min": round(per_dec[0], 2)}}
    log(f"timed {args.steps} steps: wall {wall * 1e3:.2f} ms; chunkwise {t_chunk * 1e6:.1f} us, decode {t_dec * 1e6:.1f} us")

    cf = chunk_flops(w.B, w.H, w.N, w.dk, w.dv, C)
    cb = chunk_bytes(w.B, w.H, w.N, w.dk, w.dv) + w.B * w.H * w.dk * w.dv * 4  # + the fp32 final state, written once
    db = decode_bytes(d.B, d.H, d.dk, d.dv)
    chunk_tflops = cf / t_chunk / 1e12
    tokens_per_s = w.B * w.N / t_chunk
    dec_gbps = db / t_dec / 1e9

    # The decode kernel is the longest single kernel of a step and is launched alone by its call, so
    # the events around the call time exactly that kernel.
    dec_traffic = read_counters("recurrent_step_kernel_decode_b128_h16_dk256_dv512_pmc.txt",
                                ["linear_recurrent_sequence_chunkwise_amd/csrc/recurrent_step.hip",
                                 "linear_recurrent_sequence_chunkwise_amd/csrc/common.hpp"])
    roofline = {"kernel": "recurrent_step_kernel (decode step, 128 x 16 states)", "bound": "hbm",
                "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": dec_traffic,
                "algorithmic_bytes_per_launch": db, "avg_launch_us": round(t_dec * 1e6, 2)}
    ch_traffic = read_counters("chunkwise_layer_b1_h16_n8192_pmc.txt",
                               ["linear_recurrent_sequence_chunkwise_amd/csrc/chunkwise_bf16.hip",
                                "linear_recurrent_sequence_chunkwise_amd/csrc/common.hpp"])
    roofline_chunk = {"kernel": "chunkwise forward call (scores, chunk, GroupNorm kernels)", "bound": "hbm",
                      "achieved": round(cb / t_chunk / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(cb / t_chunk / 1e9 / HBM_PEAK_GBPS, 4), "traffic": ch_traffic,
                      "mfma_bf16_tflops": round(chunk_tflops, 2), "mfma_bf16_peak": BF16_MFMA_PEAK_TFLOPS,
                      "mfma_frac": round(chunk_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                      "algorithmic_flops_per_launch": cf, "algorithmic_bytes_per_launch": cb,
                      "avg_launch_us": round(t_chunk * 1e6, 2)}

    # ---- the next rows, outside the step: swish gate after GroupNorm, chunkwise backward
    gate = (torch.randn((w.B, w.H, w.N, w.dv), generator=torch.Generator().manual_seed(7)) * 1.0).to(torch.bfloat16).to(dev)
    gn_g = R.GroupNorm(w.eps, gate=gate)
    plain = lambda: R.chunkwise_fwd(q, k, v, gam, C, groupnorm=gn, out=out, state_out=st_out, workspace=ws, stream=stream)
    tb_gate, t_gate = time_pair(plain, lambda: R.chunkwise_fwd(q, k, v, gam, C, groupnorm=gn_g, out=out, state_out=st_out,
                                                               workspace=ws, stream=stream), args.steps, stream, torch)
    del gate
    rot = R.Rotation(10000.0, 0)
    rws = torch.empty(R.workspace_bytes(R.RET_FN_CHUNKWISE, w.B, w.H, w.N, w.dk, w.dv, torch.bfloat16, torch.bfloat16, C, True,
                                        rotation=True), dtype=torch.uint8, device=dev)
    tb_rot, t_rot = time_pair(plain, lambda: R.chunkwise_fwd(q, k, v, gam, C, groupnorm=gn, rotation=rot, out=out,
                                                             state_out=st_out, workspace=rws, stream=stream),
                              args.steps, stream, torch)
    del rws
    drot = R.Rotation(10000.0, I.DECODE_PREFILL_TOKENS)
    dws = torch.empty(R.workspace_bytes(R.RET_FN_RECURRENT_STEP, d.B, d.H, 1, d.dk, d.dv, torch.bfloat16, torch.float32, 0,
                                        rotation=True), dtype=torch.uint8, device=dev)
    tb_drot, t_drot = time_pair(lambda: R.recurrent_step(qn, kn, vn, dgam, state, out=dout, stream=stream),
                                lambda: R.recurrent_step(qn, kn, vn, dgam, state, rotation=drot, out=dout, workspace=dws,
                                                         stream=stream), args.steps, stream, torch)
    # residual linear attention at the layer shape: 512-token window, softmax feature map
    rla_ws = torch.empty(R.workspace_bytes(R.RET_FN_RLA, w.B, w.H, w.N, w.dk, w.dv, torch.bfloat16, torch.float32, C),
                         dtype=torch.uint8, device=dev)
    rla_out = torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.float32, device=dev)
    t_rla = time_calls(lambda: R.rla_fwd(q, k, v, RLA_WINDOW, C, out=rla_out, state_out=st_out, workspace=rla_ws, stream=stream),
                       args.steps, stream, torch)
    del rla_ws, rla_out
    # the parallel form of the same layer (quadratic: every causal pair of the 8192 tokens)
    t_par = time_calls(lambda: R.parallel_fwd(q, k, v, gam, groupnorm=gn, out=out, stream=stream), max(2, args.steps // 4),
                       stream, torch)
    par_flops = 2 * (w.dk + w.dv) * w.B * w.H * w.N * (w.N + 1) // 2
    gdo = (torch.randn((w.B, w.H, w.N, w.dv), generator=torch.Generator().manual_seed(8))).to(torch.bfloat16).to(dev)
    bws = torch.empty(R.workspace_bytes(R.RET_FN_CHUNKWISE_BWD, w.B, w.H, w.N, w.dk, w.dv, torch.bfloat16, torch.float32, C),
                      dtype=torch.uint8, device=dev)
    t_bwd = time_calls(lambda: R.chunkwise_bwd(q, k, v, gam, gdo, C, want=("dq", "dk", "dv"), workspace=bws, stream=stream),
                       args.steps, stream, torch)
    del bws, gdo
    bf = backward_flops(w.B, w.H, w.N, w.dk, w.dv, C)
    # bf16 q, k, v, dout read; fp32 dq, dk, dv written
    bb = w.B * w.H * w.N * (2 * w.dk + 2 * w.dv) * 2 + w.B * w.H * w.N * (2 * w.dk + w.dv) * 4
    bwd_traffic = read_counters("chunkwise_backward_b1_h16_n8192_pmc.txt",
                                ["linear_recurrent_sequence_chunkwise_amd/csrc/backward.hip",
                                 "linear_recurrent_sequence_chunkwise_amd/csrc/chunkwise_bf16.hip",
                                 "linear_recurrent_sequence_chunkwise_amd/csrc/common.hpp"])
    log(f"gated chunkwise {t_gate * 1e6:.1f} us; rotated chunkwise {t_rot * 1e6:.1f} us; rotated decode {t_drot * 1e6:.1f} us; "
        f"rla {t_rla * 1e6:.1f} us; backward {t_bwd * 1e6:.1f} us")

    # cold cache: 512 MiB written before each call evicts the 256 MB MALL (and the L2s); events
    # around the chunkwise call only
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    cold = []
    for i in range(args.steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plain()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    cold.sort()
    timing["chunkwise_cold_us"] = {"mean": round(sum(cold) / len(cold), 2), "median": round(cold[len(cold) // 2], 2),
                                   "min": round(cold[0], 2)}

    # long context: N = 65536, chunk 64 .. 512, fp32 out (no GroupNorm), one call timed per chunk size
    # after a warm-up call, over max(3, K / 4) calls
    lc = I.WORKLOADS["retention_b1_h16_n65536_dk256_dv512_bf16"]
    # drawn on the device (the same distribution; 1e9 values would take the host tens of seconds)
    lq, lk, lv = I.make_qkv(lc.B, lc.H, lc.N, lc.dk, lc.dv, "bf16", seed=lc.seed, device=dev)
    lout = torch.empty((lc.B, lc.H, lc.N, lc.dv), dtype=torch.float32, device=dev)
    lst = torch.empty((lc.B, lc.H, lc.dk, lc.dv), dtype=torch.float32, device=dev)
    long_ctx = {"workload": "B=1 H=16 N=65536 d_k=256 d_v=512, bf16 in (drawn on the device), fp32 out, no GroupNorm",
                "by_chunk": {}}
    for lC in lc.chunks:
        lws = torch.empty(R.workspace_bytes(R.RET_FN_CHUNKWISE, lc.B, lc.H, lc.N, lc.dk, lc.dv, torch.bfloat16, torch.float32, lC),
                          dtype=torch.uint8, device=dev)
        t_l = time_calls(lambda: R.chunkwise_fwd(lq, lk, lv, lc.gamma_list(), lC, out=lout, state_out=lst, workspace=lws,
                                                 stream=stream), max(3, args.steps // 4), stream, torch)
        lf = chunk_flops(lc.B, lc.H, lc.N, lc.dk, lc.dv, lC)
        long_ctx["by_chunk"][str(lC)] = {"us": round(t_l * 1e6, 1), "tflops": round(lf / t_l / 1e12, 2),
                                         "tokens_per_s": round(lc.B * lc.N / t_l, 1)}
        del lws
    del lq, lk, lv, lout, lst
    peaks = measured_peaks(torch, dev, stream)
    log(f"cold chunkwise median {timing['chunkwise_cold_us']['median']:.1f} us; long context {long_ctx['by_chunk']}; peaks {peaks}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        threads = orc.threads()
        qc, kc, vc = I.make_workload_qkv(w)
        # passes over the whole layer until at least 10 s of CPU time have been spent (at least 2)
        passes, t1 = 0, time.perf_counter()
        while passes < 2 or time.perf_counter() - t1 < 10.0:
            ref, _ = orc.recurrent(qc, kc, vc, gam, want_state=False)
            orc.groupnorm(ref, w.eps)
            passes += 1
        total = time.perf_counter() - t1
        tc = total / passes
        cpu = {"value": round(cf / tc / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole N=8192 layer workload (16 heads x 8192 tokens, recurrent form + GroupNorm, fp64), "
                         f"{passes} passes in {total:.1f} s, {tc:.2f} s each; rate counted with the same chunkwise "
                         "algorithmic FLOPs",
               "tokens_per_s": round(w.B * w.N / tc, 1), "affinity_cores": len(os.sched_getaffinity(0)),
               "cpu_model": cpu_model()}
        log(f"oracle: {passes} passes, {tc:.2f} s each on {threads} threads")

    line = {
        "metric": METRIC, "value": round(chunk_tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "retention_b1_h16_n8192_dk256_dv512_bf16_gn (chunk 128, GroupNorm, bf16 out) + "
                               "decode_b128_h16_dk256_dv512 (fp32 state)",
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "tokens_per_s": round(tokens_per_s, 1), "chunkwise_us": round(t_chunk * 1e6, 2),
        "decode_GBps": round(dec_gbps, 1), "decode_us": round(t_dec * 1e6, 2),
        "decode_tokens_per_s": round(d.B / t_dec, 1),
        "roofline": roofline,
        "roofline_chunkwise": roofline_chunk,
        "swish_gate": {"chunkwise_gated_us": round(t_gate * 1e6, 2), "gate_extra_us": round((t_gate - tb_gate) * 1e6, 2)},
        "rotation": {"chunkwise_rotated_us": round(t_rot * 1e6, 2), "rotation_extra_us": round((t_rot - tb_rot) * 1e6, 2),
                     "decode_rotated_us": round(t_drot * 1e6, 2), "decode_rotation_extra_us": round((t_drot - tb_drot) * 1e6, 2)},
        "parallel": {"workload": "parallel form of the chunkwise workload (GroupNorm, bf16 out)", "us": round(t_par * 1e6, 1),
                     "tflops": round(par_flops / t_par / 1e12, 3), "algorithmic_flops": par_flops,
                     "mfma_frac": round(par_flops / t_par / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "rla": {"workload": f"residual linear attention, B=1 H=16 N=8192 d_k=256 d_v=512, window {RLA_WINDOW}, softmax "
                            "feature map, chunk 128, fp32 out", "us": round(t_rla * 1e6, 2),
                "tflops": round(cf / t_rla / 1e12, 3), "tokens_per_s": round(w.B * w.N / t_rla, 1)},
        "backward": {"workload": "dq, dk, dv of the chunkwise workload (bf16 dout, fp32 gradients)",
                     "us": round(t_bwd * 1e6, 2), "tflops": round(bf / t_bwd / 1e12, 3), "algorithmic_flops": bf,
                     "mfma_frac": round(bf / t_bwd / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                     "algorithmic_bytes": bb, "traffic": bwd_traffic,
                     "tokens_per_s": round(w.B * w.N / t_bwd, 1)},
        "timing": timing,
        "long_context": long_ctx,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "pages_context": PAGES_CONTEXT,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
