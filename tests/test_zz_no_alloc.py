"""sdpa_decode_noalloc, the allocation-free decode entry point, against sdpa_decode.

The two share their kernels; the only difference is where the split partials live (the
library's device scratch instead of the caller's workspace). Two calls in a row, the second on a
smaller input (fewer sequences, a shorter cache, several query tokens), each compared with
sdpa_decode bit for bit and with the fp64 oracle at the bf16 bar. Outputs and sdpa_decode's
workspace are NaN-filled first, so a partial the scratch call fails to write shows up.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, assert_close, nan_like, oracle_pool
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu
f32 = workloads.bf16_to_f32


def _decode_case(d):
    B, T, Hq, D = d.q.shape
    q = dev(d.q, "bf16")
    kc, vc = dev(d.k_cache, "bf16"), dev(d.v_cache, "bf16")
    kvl = dev(d.kv_lengths, "i32")
    sa.kv_cache_update(kc, vc, dev(d.k_new, "bf16"), dev(d.v_new, "bf16"), dev(d.write_index, "i32"))
    need = sa.decode_workspace_bytes(q, kc, 0)
    assert need <= sa.decode_noalloc_max_scratch_bytes()
    ref = sa.sdpa_decode(q, kc, vc, kvl, scale=d.scale, out=nan_like((B, T, Hq, D), torch.float32),
                         workspace=nan_like((need,), torch.uint8))
    got = sa.sdpa_decode_noalloc(q, kc, vc, kvl, nan_like((B, T, Hq, D), torch.float32), scale=d.scale)
    torch.cuda.synchronize()
    assert torch.equal(torch.isnan(got), torch.isnan(ref))
    assert torch.equal(torch.nan_to_num(got, nan=3.0), torch.nan_to_num(ref, nan=3.0))
    ekc, evc = oracle.kv_cache_update(d.k_cache, d.v_cache, d.k_new, d.v_new, d.write_index)
    L = d.kv_lengths
    jobs = [(lambda b=b: oracle.sdpa(f32(d.q[b:b + 1]), f32(ekc[b:b + 1, :L[b]]), f32(evc[b:b + 1, :L[b]]),
                                     scale=d.scale, is_causal="bottom_right")[0]) for b in range(B)]
    assert_close(got.cpu().numpy(), np.stack(oracle_pool(jobs)), "bf16", f"noalloc decode B{B} T{T} Hq{Hq}")


def test_noalloc_decode_two_calls_second_smaller(lib):
    say("noalloc decode: the GQA decode workload (B64 Hq32 Hkv8 D128 cap 8192)")
    _decode_case(workloads.gqa_decode())
    say("noalloc decode: then B5 Hq8 Hkv2 cap 700, 3 query tokens (some rows see no key)")
    _decode_case(workloads.gqa_decode(B=5, Hq=8, Hkv=2, D=128, capacity=700, kv_min=1, kv_max=700, base=77, q_len=3))
