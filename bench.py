"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-calibration]

A step is one causal bf16 prefill (batch 4, 16 heads, head dim 128, 4096 queries over 4096
keys, scale 1/sqrt(128)) through sdpa_fwd: one launch of the MFMA forward kernel. Inputs are
seeded N(0,1) draws rounded to bf16 (workloads.causal_prefill), resident in HBM before timing.
W untimed steps, then exactly K timed steps between two device synchronizations. The headline
``value`` is algorithmic TFLOP/s: 4 * D flops per allowed (query, key) pair, i.e. the exact
causal count B*H*L*(L+1)/2 pairs (diagonal-tile work is not credited).

The same run times the GQA decode step (batch 64, 32 query heads over 8 K/V heads, head dim
128, cache capacity 8192, kv_lengths ~ U{1024..8192}): kv_cache_update at kv_len-1, then
sdpa_decode. Its metric is KV-read GB/s: the algorithmic bytes are the K and V rows of the
attended keys, sum_b kv_len_b * Hkv * D * 2 bytes * 2, plus q and the output.

It also times the bias + block-sparse mask workload (B2 H16 D64 L8192, 2 GiB ALiBi bias, mask
through block info) and the long-context chunk (32/8 heads, 2048 queries at offset 129024 over
131072 keys), the gradient of the same prefill (sdpa_bwd: dq, dk, dv and dscale from the saved
output and log-sum-exp), in TFLOP/s over 10 * D flops per allowed pair, and the block info of
the 8192 x 8192 runtime mask from bytes and from packed bits.

Timing. The GPU's clocks take some 10-20 ms of sustained work to ramp up after the idle
seconds of input generation. Before the counted --warmup launches of every section, the same
step therefore runs for --prewarm-ms milliseconds of wall time (default 200); the count and the
time are reported (``timing.prewarm_ms``, ``timing.prewarm_launches``). The timed region is
exactly --steps launches back to back between two device synchronizations, with an event
recorded on the launch stream after each launch, so the line also carries the per-launch
median and the mean of the first and the last quarter of the window. The prefill section also
times launches one at a time with 512 MiB written between them (the 256 MiB last-level cache
flushed), reported as ``timing.mall_flushed_median_ms`` beside the back-to-back figure.

Measured peaks. Two probes of the library (sdpa_measure_mfma_bf16: only bf16 MFMAs, two waves
per SIMD; sdpa_measure_stream_read: a 4 GiB nontemporal streaming read) give the rates the chip
sustains;
every roofline carries its fraction of the vendor peak (``frac``) and of the measured one
(``frac_of_measured``).

Printed: one JSON line (rank 0) with the contract fields, a ``roofline`` object for the
prefill kernel (achieved = algorithmic flops per launch / average launch time measured with
HIP events on the launch stream; peak = 2500 TFLOP/s bf16 dense MFMA), a ``decode`` object with
its own roofline against 8000 GB/s, a sampled parity check of the timed outputs against the
fp64 oracle, and ``cpu_baseline``: the oracle timed on this host's cores on a bounded sample.
"""
import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PREFILL_COUNTERS = (os.path.join(ROOT, "profiles", "fwd_mfma_causal_b4h16d128l4096_counters.txt"),
                    os.path.join(ROOT, "transformer_attention_sdpa_amd", "csrc", "fwd_mfma.hip"))
DECODE_COUNTERS = (os.path.join(ROOT, "profiles", "decode_gqa_b64h32kv8d128_counters.txt"),
                   os.path.join(ROOT, "transformer_attention_sdpa_amd", "csrc", "decode.hip"))
BIAS_MASK_COUNTERS = (os.path.join(ROOT, "profiles", "fwd_mfma_bias_block_mask_b2h16d64l8192.md"),
                      os.path.join(ROOT, "transformer_attention_sdpa_amd", "csrc", "fwd_mfma.hip"))
BACKWARD_COUNTERS = (os.path.join(ROOT, "profiles", "bwd_causal_b4h16d128l4096_counters.txt"),
                     os.path.join(ROOT, "transformer_attention_sdpa_amd", "csrc", "bwd_mfma.hip"))


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    # the clocks ramp up over 10-20 ms of sustained work: every section first runs its own step
    # for this much wall time (reported in the line), then the counted warm-up launches
    p.add_argument("--prewarm-ms", type=float, default=200.0)
    p.add_argument("--skip-peaks", action="store_true", help="skip the measured-peak probes")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU budget of the oracle baseline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (for scaling HBM byte counters)")
    p.add_argument("--skip-decode", action="store_true")
    p.add_argument("--skip-mask-info", action="store_true")
    p.add_argument("--skip-backward", action="store_true")
    p.add_argument("--skip-extra", action="store_true", help="skip the bias + block-mask and long-context timings")
    p.add_argument("--sections", default="all",
                   help="comma list of the sections to run besides the headline prefill (backward, decode, "
                        "mask_info, bias_block_mask, chunked_prefill, widened), or 'all'")
    a = p.parse_args()
    if a.sections != "all":
        want = set(a.sections.split(","))
        a.skip_backward = a.skip_backward or "backward" not in want
        a.skip_decode = a.skip_decode or "decode" not in want
        a.skip_mask_info = a.skip_mask_info or "mask_info" not in want
        a.skip_bias_mask = a.skip_extra or "bias_block_mask" not in want
        a.skip_chunked = a.skip_extra or "chunked_prefill" not in want
        a.skip_widened = a.skip_extra or "widened" not in want
    else:
        a.skip_bias_mask = a.skip_chunked = a.skip_widened = a.skip_extra
    return a


def source_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_traffic(counters):
    """HBM bytes per launch from a committed rocprofv3 counter summary (path, kernel source), if
    it was taken from the current kernel source; else None."""
    summary, source = counters
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(source):
        return None
    return float(m_bytes.group(1))


PREWARM_MS = 200.0          # set from --prewarm-ms in main()
TIMINGS = {}                # section -> per-launch statistics of its timed window


def prewarm(fn, ms):
    """Run fn back to back until `ms` of wall time have passed (the clocks ramp up under load)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= ms:
            return n, el


def time_steps(fn, steps, warmup, stream, label=None):
    """--prewarm-ms of fn, `warmup` counted launches, then exactly `steps` timed launches back to
    back on `stream`, with an event after each. Returns (seconds for all steps, wall seconds);
    the per-launch statistics go to TIMINGS[label]."""
    import torch
    pw_n, pw_ms = prewarm(fn, PREWARM_MS)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    q = max(1, steps // 4)
    if label:
        TIMINGS[label] = {"prewarm_ms": round(pw_ms, 1), "prewarm_launches": pw_n, "warmup": warmup,
                          "median_ms": round(float(sorted(per)[len(per) // 2]), 4),
                          "first_quarter_ms": round(sum(per[:q]) / q, 4),
                          "last_quarter_ms": round(sum(per[-q:]) / q, 4)}
    return ev[0].elapsed_time(ev[-1]) / 1e3, wall


def time_flushed(fn, n, stream, flush_bytes=512 << 20):
    """Median milliseconds of `n` single launches, each after `flush_bytes` written to a scratch
    buffer (more than the 256 MiB last-level cache holds), timed by events around the launch."""
    import torch
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):                      # queued back to back: the GPU never idles in between
        buf.fill_(i & 255)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) for e0, e1 in ev]
    del buf
    return float(sorted(times)[n // 2])


def measured_peaks(stream):
    """The bf16 MFMA rate and the HBM streaming-read rate this GPU sustains, from the library's
    two probes (median of 5 timed launches each, after a time-based warm-up)."""
    import torch
    import transformer_attention_sdpa_amd as sa
    res = {}
    wgs, iters = 512, 20000                        # 2 workgroups per CU: two waves per SIMD
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    flops = [0.0]

    def mf():
        flops[0] = sa.measure_mfma_bf16(wgs, iters, sink)
    prewarm(mf, PREWARM_MS)
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mf()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    t = sorted(ts)[2]
    res["mfma_bf16_tflops"] = round(flops[0] / t / 1e12, 1)
    res["mfma_probe"] = f"{wgs} workgroups x 4 waves x {iters} x 4 v_mfma_f32_32x32x16_bf16, median of 5"
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    ssink = torch.empty(16384 * 4, dtype=torch.int32, device="cuda")
    nb = [0]

    def rd():
        nb[0] = sa.measure_stream_read(buf, 16384, ssink)
    prewarm(rd, PREWARM_MS)
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rd()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    t = sorted(ts)[2]
    res["hbm_read_gbs"] = round(nb[0] / t / 1e9, 1)
    res["read_probe"] = "4 GiB streaming read, 16-byte nontemporal loads, 16384 workgroups of 256, median of 5"
    del buf, ssink, sink
    torch.cuda.empty_cache()
    return res


def oracle_rows_parity(out, w, rows):
    import numpy as np
    import oracle
    got = out[:, rows].float().cpu().numpy().astype(np.float64)
    ref = oracle.sdpa(w.values("q"), w.values("k"), w.values("v"), scale=w.scale, is_causal=w.is_causal,
                      q_offset=w.q_offset, rows=rows)
    d = got - ref
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / np.linalg.norm(ref))


def backward_parity(w, q, k, v, outb, dout, lse, grads):
    """The timed gradients of two (batch, head) slices against the fp64 oracle gradient of
    those slices (each slice is an independent attention: one K/V head per query head)."""
    import numpy as np
    import torch
    import oracle
    import workloads
    import transformer_attention_sdpa_amd as sa
    sa.sdpa_bwd(q, k, v, outb, dout, lse, is_causal=True, scale=w.scale, grads=grads)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    worst = {}
    do_np = workloads.widen(workloads.output_cotangent(w, 7), "bf16")
    for b, h in ((0, 0), (w.q.shape[0] - 1, w.q.shape[2] - 1)):
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        ref = oracle.sdpa_grad(sl(w.values("q")), sl(w.values("k")), sl(w.values("v")), sl(do_np),
                               scale=w.scale, is_causal=True)
        for n, t in zip(("dq", "dk", "dv"), grads[:3]):
            got = f(t[b:b + 1, :, h:h + 1])
            mag = max(1.0, float(np.max(np.abs(ref[n]))))
            d = got - ref[n]
            m, r = float(np.max(np.abs(d))) / mag, float(np.linalg.norm(d) / np.linalg.norm(ref[n]))
            worst[n] = [max(worst.get(n, [0, 0])[0], m), max(worst.get(n, [0, 0])[1], r)]
    return {"slices_checked": "(b, h) = (0, 0) and (B-1, H-1), every row",
            **{n: {"max_abs_over_mag": v[0], "rel_l2": v[1]} for n, v in worst.items()},
            "bar": "max_abs/max(1,|ref|) <= 2e-2, rel_l2 <= 5e-3"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_prefill(w, budget_s):
    """The fp64 oracle on whole (batch, head) pairs of the prefill workload until the budget is spent."""
    import numpy as np
    import oracle
    B, Lq, Lkv, Hq, Hkv, D, Dv = w.shape
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    done, t_total = 0, 0.0
    pairs = [(b, h) for b in range(B) for h in range(Hq)]
    for (b, h) in pairs:
        t0 = time.perf_counter()
        oracle.sdpa(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], scale=w.scale,
                    is_causal=True)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    flops = 4.0 * D * (Lq * (Lq + 1) / 2) * done
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {B * Hq} (batch, head) pairs, all {Lq} query rows each, fp64 numpy",
            "seconds": round(t_total, 2), "cpu_model": cpu_model(),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "cores_note": "cores = the BLAS threads the oracle's matrix products ran on"}


def progress(msg):
    """One line on stderr per finished section: the JSON result stays the only stdout line."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads
    import transformer_attention_sdpa_amd as sa

    global PREWARM_MS
    PREWARM_MS = args.prewarm_ms
    sa.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    peaks = None if args.skip_peaks else measured_peaks(stream)
    progress("measured peaks done" if peaks else "measured peaks skipped")

    def frac_measured(achieved, key):
        return round(achieved / peaks[key], 4) if peaks else None

    # ---- causal prefill -------------------------------------------------------------------
    w = workloads.causal_prefill()
    B, Lq, Lkv, Hq, Hkv, D, Dv = w.shape
    q, k, v = (sa.from_numpy(getattr(w, n), "bf16") for n in ("q", "k", "v"))
    out = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device="cuda")
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step = lambda: sa.sdpa(q, k, v, is_causal=True, scale=w.scale, out=out)
    t_gpu, t_wall = time_steps(step, args.steps, args.warmup, stream, "prefill")
    TIMINGS["prefill"]["mall_flushed_median_ms"] = round(time_flushed(step, 10, stream), 4)
    pairs = B * Hq * Lq * (Lq + 1) / 2
    flops = 4.0 * D * pairs
    per_launch = t_gpu / args.steps
    tflops = flops / per_launch / 1e12
    rows = [0, 1, 127, 128, 1000, 2047, 2048, 3333, 4094, 4095]
    p_max, p_rel = oracle_rows_parity(out, w, rows)
    result = {
        "metric": "attention TFLOP/s (causal bf16 prefill) + decode KV-read GB/s, 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_launch * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {"workload": "causal_prefill", "batch": B, "heads": Hq, "head_dim": D, "q_len": Lq,
                   "kv_len": Lkv, "is_causal": True, "scale": w.scale, "out_dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": counters_traffic(PREFILL_COUNTERS),
                     "kernel": "fwd_mfma_kernel<128,0,0>", "flops_per_launch": flops,
                     "path": sa.sdpa_fwd_path(q, k, v, is_causal=True, scale=w.scale),
                     "measured_peak": peaks["mfma_bf16_tflops"] if peaks else None,
                     "frac_of_measured": frac_measured(tflops, "mfma_bf16_tflops")},
        "timing": TIMINGS["prefill"],
        "measured_peaks": peaks,
        "parity": {"rows_checked": f"{len(rows)} query rows x {B * Hq} (batch, head)", "max_abs": p_max,
                   "rel_l2": p_rel, "bar": "max_abs <= 2e-2, rel_l2 <= 5e-3 (bf16 output)"},
        "wall_s_timed_region": round(t_wall, 4),
    }
    progress("prefill timed")
    # ---- gradient (sdpa_bwd) of the same causal prefill ------------------------------------
    # one call: prep (D = rowsum(dO * O)), dK/dV, dQ and the dscale sum. Algorithmic work: the
    # five products per allowed pair (S again, dP, dV, dK, dQ), 10 * D flops, 2.5x the forward.
    if not args.skip_backward:
        out32, lse = sa.sdpa(q, k, v, is_causal=True, scale=w.scale, out_dtype=torch.float32, return_lse=True)
        outb = out32.to(torch.bfloat16)
        dout = sa.from_numpy(workloads.output_cotangent(w, 7), "bf16")
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty(1, dtype=torch.float32, device="cuda"))
        # the workspace with room for the stored dS: the dK/dV pass writes dS, the dQ pass reads it
        bws = torch.empty(sa.bwd_workspace_bytes(q, k, v, store_ds=True), dtype=torch.uint8, device="cuda")
        bstep = lambda: sa.sdpa_bwd(q, k, v, outb, dout, lse, is_causal=True, scale=w.scale, grads=grads,
                                    workspace=bws)
        bsteps = max(1, args.steps // 2)
        t_b, _ = time_steps(bstep, bsteps, max(1, args.warmup // 2), stream, "backward")
        flops_b = 10.0 * D * pairs
        tf_b = flops_b / (t_b / bsteps) / 1e12
        result["backward"] = {
            "metric": "attention gradient TFLOP/s (causal bf16 prefill)", "value": round(tf_b, 2),
            "unit": "TFLOP/s", "ms_per_step": round(t_b / bsteps * 1e3, 4), "steps": bsteps,
            "config": {"workload": "causal_prefill", "batch": B, "heads": Hq, "head_dim": D, "q_len": Lq,
                       "is_causal": True, "grad_dtype": "bf16", "saved_out_dtype": "bf16"},
            "roofline": {"bound": "mfma", "achieved": round(tf_b, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf_b / PEAK_BF16_TFLOPS, 4), "traffic": counters_traffic(BACKWARD_COUNTERS),
                         "path": sa.sdpa_bwd_path(q, k, v, outb, dout, is_causal=True, scale=w.scale,
                                                  workspace_bytes=bws.numel()),
                         "flops_per_call": flops_b, "frac_of_measured": frac_measured(tf_b, "mfma_bf16_tflops"),
                         "kernel": "bwd_prep + bwd_dkdv8_kernel<128> (stores dS) + bwd_dq_ds_kernel<128> + bwd_dscale"},
            "parity": backward_parity(w, q, k, v, outb, dout, lse, grads),
            "timing": TIMINGS["backward"],
        }
        del out32, outb, dout, grads, bws, lse
    del q, k, v, out
    torch.cuda.empty_cache()

    progress("gradient section done")
    # ---- GQA decode -----------------------------------------------------------------------
    if not args.skip_decode:
        d = workloads.gqa_decode()
        Bd, _, Hqd, Dd = d.q.shape
        Hkvd = d.k_cache.shape[2]
        qd = sa.from_numpy(d.q, "bf16")
        kc, vc = sa.from_numpy(d.k_cache, "bf16"), sa.from_numpy(d.v_cache, "bf16")
        kn, vn = sa.from_numpy(d.k_new, "bf16"), sa.from_numpy(d.v_new, "bf16")
        widx = sa.from_numpy(d.write_index, "i32")
        kvl = sa.from_numpy(d.kv_lengths, "i32")
        od = torch.empty((Bd, 1, Hqd, Dd), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(sa.decode_workspace_bytes(qd, kc, 0), dtype=torch.uint8, device="cuda")

        def dstep():
            sa.kv_cache_update(kc, vc, kn, vn, widx)
            sa.sdpa_decode(qd, kc, vc, kvl, scale=d.scale, out=od, workspace=ws)

        td, _ = time_steps(dstep, args.steps, args.warmup, stream, "decode_with_update")
        tdec, _ = time_steps(lambda: sa.sdpa_decode(qd, kc, vc, kvl, scale=d.scale, out=od, workspace=ws),
                             args.steps, args.warmup, stream, "decode")
        kv_bytes = float(np.sum(d.kv_lengths.astype(np.int64))) * Hkvd * Dd * 2 * 2
        io_bytes = float(Bd * Hqd * Dd * 2 * 2)
        gbs = (kv_bytes + io_bytes) / (tdec / args.steps) / 1e9
        # parity of the decode output on a few sequences
        import oracle
        f = workloads.bf16_to_f32
        sel = [0, Bd // 2, Bd - 1]
        ekc, evc = oracle.kv_cache_update(d.k_cache[sel], d.v_cache[sel], d.k_new[sel], d.v_new[sel],
                                          d.write_index[sel])
        refs = [oracle.sdpa(f(d.q[b:b + 1]), f(ekc[i:i + 1, :d.kv_lengths[b]]), f(evc[i:i + 1, :d.kv_lengths[b]]),
                            scale=d.scale, is_causal="bottom_right")[0] for i, b in enumerate(sel)]
        got = od[sel].float().cpu().numpy()
        diff = got - np.stack(refs)
        result["decode"] = {
            "metric": "decode KV-read GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_step": round(tdec / args.steps * 1e3, 4),
            "ms_per_step_with_cache_update": round(td / args.steps * 1e3, 4),
            "config": {"workload": "gqa_decode", "batch": Bd, "q_heads": Hqd, "kv_heads": Hkvd, "head_dim": Dd,
                       "capacity": d.k_cache.shape[1], "kv_lengths": "U{1024..8192} (seeded)",
                       "sum_kv_lengths": int(np.sum(d.kv_lengths))},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counters_traffic(DECODE_COUNTERS),
                         "bytes_per_step": kv_bytes + io_bytes,
                         "measured_peak": peaks["hbm_read_gbs"] if peaks else None,
                         "frac_of_measured": frac_measured(gbs, "hbm_read_gbs"),
                         "note": "split + combine kernels together (one sdpa_decode call)"},
            "timing": TIMINGS["decode"], "timing_with_update": TIMINGS["decode_with_update"],
            "parity": {"sequences_checked": sel, "max_abs": float(np.max(np.abs(diff))),
                       "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(np.stack(refs)))},
        }
        del qd, kc, vc, od, ws
        torch.cuda.empty_cache()

    progress("decode section done")
    # ---- block info of a runtime mask: bytes (U8) and packed bits (U1) --------------------
    # the 8192 x 8192 mask of the bias + block-sparse workload, 128 x 128 blocks; the bound is
    # reading the mask (64 MiB as bytes, 8 MiB as bits) plus writing the partial blocks' bits
    if not args.skip_mask_info:
        mask = workloads.block_sparse_mask(8192, 8192, 128, k=3)
        mu8 = sa.from_numpy(mask, "u8")
        mu1 = sa.PackedMask(sa.from_numpy(workloads.pack_mask_bits(mask, 1), "i32"), mask.shape[-1])
        mi = {}
        infos = {}
        for name, m in (("u8", mu8), ("u1", mu1)):
            store = sa.build_block_mask_info(m, 128, 128).storage          # reused by the timed calls
            t_mi, _ = time_steps(lambda m=m, st=store: sa.build_block_mask_info(m, 128, 128, storage=st),
                                 args.steps, args.warmup, stream, "mask_info_" + name)
            infos[name] = sa.build_block_mask_info(m, 128, 128).to_numpy()
            mask_bytes = mask.size if name == "u8" else mask.size / 8
            mi[name] = {"ms": round(t_mi / args.steps * 1e3, 4),
                        "mask_GB_per_s": round(mask_bytes / (t_mi / args.steps) / 1e9, 1)}
        same = all(np.array_equal(infos["u8"][k], infos["u1"][k])
                   for k in ("block_mask", "mask_next", "row_ptr", "data_next", "partial_bits"))
        result["mask_info"] = {"workload": "bias_block_mask mask, 1 x 1 x 8192 x 8192, 128 x 128 blocks",
                               "n_partial": int(infos["u8"]["n_partial"]), "u1_equals_u8": bool(same), **mi}
        del mu8, mu1
        torch.cuda.empty_cache()

    progress("block info section done")
    # ---- bias + block-sparse mask (B2 H16 D64 L8192) and the long-context chunk ------------
    # bias + mask: ALiBi bias [1][16][8192][8192] bf16 (2 GiB) and the runtime mask through its
    # block info; algorithmic work counts the non-empty 128 x 128 blocks (4 * D flops per pair of
    # such a block), and the bias bytes of those blocks read once. Long context: B1, 32 query
    # heads over 8 K/V heads, 2048 queries at offset 129024 over 131072 keys, causal; exact pairs.
    if not args.skip_bias_mask:
        w4 = workloads.bias_block_mask()
        B4_, Lq4, _, Hq4, _, D4, _ = w4.shape
        q4, k4, v4 = (sa.from_numpy(getattr(w4, n), "bf16") for n in ("q", "k", "v"))
        bias4 = sa.from_numpy(w4.bias, "bf16")
        info4 = sa.build_block_mask_info(sa.from_numpy(w4.mask, "u8"), 128, 128)
        nonempty = int(np.count_nonzero(info4.to_numpy()["block_mask"]))
        out4 = torch.empty((B4_, Lq4, Hq4, D4), dtype=torch.bfloat16, device="cuda")
        st4 = lambda: sa.sdpa(q4, k4, v4, bias4, None, mask_info=info4, scale=w4.scale, out=out4)
        n4 = max(2, args.steps // 2)
        t4, _ = time_steps(st4, n4, max(2, args.warmup // 2), stream, "bias_block_mask")
        fl4 = float(nonempty) * B4_ * Hq4 * 4.0 * 128 * 128 * D4
        bias_bytes = float(nonempty) * Hq4 * 128 * 128 * 2
        per4 = t4 / n4
        result["bias_block_mask"] = {
            "metric": "attention TFLOP/s over non-empty blocks", "value": round(fl4 / per4 / 1e12, 2),
            "unit": "TFLOP/s", "ms_per_step": round(per4 * 1e3, 4), "steps": n4,
            "config": {"workload": "bias_block_mask", "batch": B4_, "heads": Hq4, "head_dim": D4, "q_len": Lq4,
                       "bias": "ALiBi bf16 [1][16][8192][8192]", "mask_blocks_nonempty": nonempty,
                       "mask_blocks_total": int(info4.to_numpy()["block_mask"].size)},
            "roofline": {"bound": "mixed: MFMA and the bias stream", "mfma_frac": round(fl4 / per4 / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "bias_GB_per_s": round(bias_bytes / per4 / 1e9, 1),
                         "bias_frac_of_hbm": round(bias_bytes / per4 / 1e9 / PEAK_HBM_GBS, 4),
                         "mfma_frac_of_measured": frac_measured(fl4 / per4 / 1e12, "mfma_bf16_tflops"),
                         "traffic": counters_traffic(BIAS_MASK_COUNTERS),
                         "algorithmic_bytes": float(bias_bytes + 4.0 * B4_ * Lq4 * Hq4 * D4 * 2),
                         "note": "bias bytes of the non-empty blocks counted once (the batch shares them)"},
            "timing": TIMINGS["bias_block_mask"],
        }
        del q4, k4, v4, bias4, info4, out4
        torch.cuda.empty_cache()
    if not args.skip_chunked:
        w5 = workloads.chunked_prefill()
        B5, Lq5, Lkv5, Hq5, Hkv5, D5, _ = w5.shape
        q5, k5, v5 = (sa.from_numpy(getattr(w5, n), "bf16") for n in ("q", "k", "v"))
        out5 = torch.empty((B5, Lq5, Hq5, D5), dtype=torch.bfloat16, device="cuda")
        qo5 = int(w5.q_offset)
        st5 = lambda: sa.sdpa(q5, k5, v5, is_causal=True, q_offset=qo5, scale=w5.scale, out=out5)
        n5 = max(2, args.steps // 5)
        t5, _ = time_steps(st5, n5, max(2, args.warmup // 5), stream, "chunked_prefill")
        pairs5 = float(Lq5) * qo5 + Lq5 * (Lq5 + 1) / 2
        fl5 = 4.0 * D5 * pairs5 * Hq5 * B5
        per5 = t5 / n5
        result["chunked_prefill"] = {
            "metric": "attention TFLOP/s (long-context chunk)", "value": round(fl5 / per5 / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(per5 * 1e3, 4), "steps": n5,
            "config": {"workload": "chunked_prefill", "batch": B5, "q_heads": Hq5, "kv_heads": Hkv5, "head_dim": D5,
                       "q_len": Lq5, "kv_len": Lkv5, "q_offset": qo5, "is_causal": True},
            "roofline": {"bound": "mfma", "achieved": round(fl5 / per5 / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(fl5 / per5 / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "flops_per_launch": fl5, "frac_of_measured": frac_measured(fl5 / per5 / 1e12, "mfma_bf16_tflops")},
            "timing": TIMINGS["chunked_prefill"],
        }
        del q5, k5, v5, out5
        torch.cuda.empty_cache()

    progress("bias + block mask and long-context sections done")
    # ---- widened paths: packed sequences, several decode tokens, f16 ------------------------
    # packed: causal prefill over documents packed in one sequence (16 heads, D 128, segment
    # lengths ~ U{256..4096} up to 32768 tokens), exact in-segment causal pairs; decode: the GQA
    # decode cache with 4 new query tokens per sequence (KV bytes as for one token: each K/V row
    # is read once for all 4); f16: the causal prefill with f16 inputs (the bf16 values, exact in f16);
    # non-causal: the causal prefill's tensors with every pair allowed
    if not args.skip_widened:
        nx = {}
        rng = np.random.default_rng([1007, 11])
        lens = []
        while sum(lens) < 32768:
            lens.append(int(rng.integers(256, 4097)))
        lens[-1] -= sum(lens) - 32768
        lens = [t for t in lens if t > 0]
        tot = sum(lens)
        Hp, Dp = 16, 128
        qp_, kp_, vp_ = (sa.from_numpy(workloads.normal_tensor(np.random.default_rng([1007, tag]), (tot, Hp, Dp), "bf16"),
                                       "bf16") for tag in (0, 1, 2))
        segs = sa.from_numpy(np.array(lens, dtype=np.int32), "i32")
        outp = torch.empty((tot, Hp, Dp), dtype=torch.bfloat16, device="cuda")
        stp = lambda: sa.sdpa_packed(qp_, kp_, vp_, segs, is_causal=True, maxlen=max(lens), out=outp)
        n_p = max(2, args.steps // 2)
        t_p, _ = time_steps(stp, n_p, max(2, args.warmup), stream)
        fl_p = 4.0 * Dp * Hp * sum(t * (t + 1) / 2 for t in lens)
        nx["packed_causal_prefill"] = {"segments": len(lens), "total_tokens": tot, "heads": Hp, "head_dim": Dp,
                                       "ms": round(t_p / n_p * 1e3, 4),
                                       "TFLOP_per_s": round(fl_p / (t_p / n_p) / 1e12, 2),
                                       "frac_of_2500": round(fl_p / (t_p / n_p) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del qp_, kp_, vp_, outp
        d4 = workloads.gqa_decode(q_len=4)
        q4 = sa.from_numpy(d4.q, "bf16")
        kc4, vc4 = sa.from_numpy(d4.k_cache, "bf16"), sa.from_numpy(d4.v_cache, "bf16")
        sa.kv_cache_update(kc4, vc4, sa.from_numpy(d4.k_new, "bf16"), sa.from_numpy(d4.v_new, "bf16"),
                           sa.from_numpy(d4.write_index, "i32"))
        kvl4 = sa.from_numpy(d4.kv_lengths, "i32")
        B4d, T4, Hq4d, D4d = d4.q.shape
        o4 = torch.empty((B4d, T4, Hq4d, D4d), dtype=torch.bfloat16, device="cuda")
        ws4 = torch.empty(sa.decode_workspace_bytes(q4, kc4, 0), dtype=torch.uint8, device="cuda")
        std = lambda: sa.sdpa_decode(q4, kc4, vc4, kvl4, scale=d4.scale, out=o4, workspace=ws4)
        t_d4, _ = time_steps(std, args.steps, args.warmup, stream)
        by4 = float(np.sum(d4.kv_lengths.astype(np.int64))) * d4.k_cache.shape[2] * D4d * 2 * 2 + \
            2.0 * B4d * T4 * Hq4d * D4d * 2
        nx["decode_4_tokens"] = {"batch": B4d, "q_tokens": T4, "q_heads": Hq4d, "kv_heads": int(d4.k_cache.shape[2]),
                                 "ms": round(t_d4 / args.steps * 1e3, 4),
                                 "GB_per_s": round(by4 / (t_d4 / args.steps) / 1e9, 1),
                                 "frac_of_8000": round(by4 / (t_d4 / args.steps) / 1e9 / PEAK_HBM_GBS, 4)}
        del q4, kc4, vc4, o4, ws4
        torch.cuda.empty_cache()
        q16, k16, v16 = (sa.from_numpy(getattr(w, n), "bf16").to(torch.float16) for n in ("q", "k", "v"))
        o16 = torch.empty((B, Lq, Hq, D), dtype=torch.float16, device="cuda")
        st16 = lambda: sa.sdpa(q16, k16, v16, is_causal=True, scale=w.scale, out=o16)
        t16, _ = time_steps(st16, args.steps, args.warmup, stream)
        nx["f16_causal_prefill"] = {"workload": "causal_prefill in f16", "ms": round(t16 / args.steps * 1e3, 4),
                                    "TFLOP_per_s": round(flops / (t16 / args.steps) / 1e12, 2),
                                    "frac_of_2500": round(flops / (t16 / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del q16, k16, v16, o16
        torch.cuda.empty_cache()
        # the same tensors without the causal limit: every (query, key) pair, 4 * D flops each
        qn, kn, vn = (sa.from_numpy(getattr(w, n), "bf16") for n in ("q", "k", "v"))
        ond = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device="cuda")
        stn = lambda: sa.sdpa(qn, kn, vn, is_causal=False, scale=w.scale, out=ond)
        tnd, _ = time_steps(stn, args.steps, args.warmup, stream)
        fl_nd = 4.0 * D * B * Hq * Lq * Lkv
        nx["noncausal_prefill"] = {"workload": "causal_prefill shapes, is_causal false", "ms": round(tnd / args.steps * 1e3, 4),
                                   "TFLOP_per_s": round(fl_nd / (tnd / args.steps) / 1e12, 2),
                                   "frac_of_2500": round(fl_nd / (tnd / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del qn, kn, vn, ond
        torch.cuda.empty_cache()
        result["widened"] = nx

    progress("widened sections done")
    # ---- CPU baseline (rank 0, N = 1 only) ------------------------------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
