"""KV-cache update at a write index (oracle; test infrastructure only).

Sources: the keras issue "MultiHeadAttention is missing a position_bias call argument,
making Alibi or T5-style position embedding impossible to implement" (the proposal of
separate key and value caches with an index that says where the new keys and values
go), and the Flax discussion "is MultiHeadAttention in flax.nnx JIT-compilable with the
decode=True parameter?" (a cache laid out [batch, position, head, feature] that grows by
one position per decode step).

Row t of the new keys/values of batch element b goes to cache position
write_index[b] + t. Positions outside [0, capacity) are not written (the pages say
nothing about them; skipping keeps every write in bounds).
"""
import numpy as np


def kv_cache_update(k_cache, v_cache, k_new, v_new, write_index):
    """Return updated copies of the caches.

    k_cache, v_cache: [B][capacity][Hkv][D]; k_new, v_new: [B][T][Hkv][D];
    write_index: [B] integers. Works on any dtype (bf16 bit patterns included): it copies.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, capacity = kc.shape[0], kc.shape[1]
    T = k_new.shape[1]
    for b in range(B):
        for t in range(T):
            pos = int(write_index[b]) + t
            if 0 <= pos < capacity:
                kc[b, pos] = k_new[b, t]
                vc[b, pos] = v_new[b, t]
    return kc, vc
