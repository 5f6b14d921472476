"""Helpers for the GPU parity tests: move a seeded workload to the device, run the HIP path
through the binding, run the oracle on the same values, and compare to the stated bar.

Bar (floating point): fp32 inputs max-abs <= 1e-5; bf16 inputs (fp32 accumulate) max-abs
<= 2e-2 and relative L2 <= 5e-3, both over the finite entries; NaN positions must match
exactly. Integer/byte results are compared bit for bit.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads
import transformer_attention_sdpa_amd as sa

# f16 inputs take the bf16 bar: 16-bit inputs, fp32 accumulation (f16 rounds more finely)
TOL = {"f32": dict(max_abs=1e-5, rel_l2=None), "bf16": dict(max_abs=2e-2, rel_l2=5e-3),
       "f16": dict(max_abs=2e-2, rel_l2=5e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return sa.from_numpy(a, dtype, "cuda")


def gpu_inputs(w: workloads.Attention):
    t = {"q": dev(w.q, w.dtype), "k": dev(w.k, w.dtype), "v": dev(w.v, w.dtype)}
    t["bias"] = dev(w.bias, w.bias_dtype) if w.bias is not None else None
    t["mask"] = dev(w.mask, "u8") if w.mask is not None else None
    return t


def per_batch(x):
    if x is None or isinstance(x, (int, np.integer)):
        return x
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


def run_gpu(w: workloads.Attention, out_dtype=torch.float32, use_mask_info=False, bq=128, bkv=128,
            q_lengths=None, t=None):
    t = t or gpu_inputs(w)
    info = None
    if use_mask_info and t["mask"] is not None:
        info = sa.build_block_mask_info(t["mask"], bq, bkv)
    out = sa.sdpa(t["q"], t["k"], t["v"], t["bias"], None if info else t["mask"], mask_info=info,
                  scale=w.scale, is_causal=w.is_causal, q_offset=per_batch(w.q_offset),
                  kv_lengths=per_batch(w.kv_lengths), q_lengths=per_batch(q_lengths), qk_norm=w.qk_norm,
                  out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def run_oracle(w: workloads.Attention, rows=None, q_lengths=None):
    return oracle.sdpa(w.values("q"), w.values("k"), w.values("v"), bias=w.values("bias"), mask=w.mask,
                       scale=w.scale, is_causal=w.is_causal, q_offset=w.q_offset, kv_lengths=w.kv_lengths,
                       q_lengths=q_lengths, qk_norm=w.qk_norm, rows=rows)


def metrics(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"NaN positions differ: gpu {nan_g.sum()} vs oracle {nan_r.sum()}"
    fin = ~nan_r
    if not fin.any():
        return 0.0, 0.0
    d = got[fin] - ref[fin]
    max_abs = float(np.max(np.abs(d)))
    nref = float(np.linalg.norm(ref[fin]))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, dtype, label=""):
    max_abs, rel = metrics(got, ref)
    tol = TOL[dtype]
    say(f"  {label}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= tol["max_abs"], f"{label}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{label}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


def assert_grad_close(got, ref, dtype, label=""):
    """The bar above, for a gradient: max-abs taken relative to max(1, max |oracle|), since a
    gradient sums over many pairs and has no fixed magnitude; rel-L2 as for the output."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite gradient entries"
    mag = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    d = got - ref
    max_abs = float(np.max(np.abs(d))) / mag if ref.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    tol = TOL[dtype]
    say(f"  {label}: max_abs/mag={max_abs:.3e} (mag {mag:.2f}) rel_l2={rel:.3e}")
    assert max_abs <= tol["max_abs"], f"{label}: max-abs/mag {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{label}: rel-L2 {rel:.3e} > {tol['rel_l2']}"


def oracle_pool(jobs, workers=None):
    """Results of the zero-argument oracle calls ``jobs``, run on a thread pool with one BLAS
    thread per worker (numpy releases the GIL in its matrix products and element loops). The
    pool is sized to the host's cores, at most 16."""
    from threadpoolctl import threadpool_limits
    n = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(n) as ex:
            return list(ex.map(lambda f: f(), jobs))


def nan_like(shape, dtype, device="cuda"):
    """A tensor filled with NaN (floating dtypes) or 0xFF bytes (uint8), to poison an output or a
    workspace: any element a kernel fails to write stays NaN and fails the comparison."""
    if dtype == torch.uint8:
        return torch.full(shape, 0xFF, dtype=dtype, device=device)
    return torch.full(shape, float("nan"), dtype=dtype, device=device)
