"""Algorithmic work of the attention core: the flops and bytes the method itself
must do, used for throughput and roofline figures (never the dense T x T work a
tiled kernel may skip or the masked entries it may compute)."""


def prefill_pairs(lengths):
    """Unmasked (query, key) pairs per query head: sum of L(L+1)/2."""
    return sum(int(L) * (int(L) + 1) // 2 for L in lengths)


def prefill_flops(lengths, n_q_heads, head_dim=128):
    """2*d flops for the score and 2*d for the P.V product per unmasked pair,
    per query head: sum over sequences of 2 * d * Hq * L * (L + 1)."""
    return 4 * head_dim * n_q_heads * prefill_pairs(lengths)


def kv_bytes_per_token(n_kv_heads, head_dim=128, elem_bytes=2, layers=1):
    """K and V bytes one cached token occupies (2 x layers x Hkv x d x bytes)."""
    return 2 * layers * n_kv_heads * head_dim * elem_bytes


def decode_kv_read_bytes(cached_lengths, n_kv_heads, head_dim=128, elem_bytes=2):
    """Cache bytes one decode step must read: K and V of the L_i cached tokens
    plus the new token's own K and V (written to the cache, read back)."""
    per_tok = kv_bytes_per_token(n_kv_heads, head_dim, elem_bytes)
    return sum((int(L) + 1) * per_tok for L in cached_lengths)


def decode_total_bytes(cached_lengths, n_q_heads, n_kv_heads, head_dim=128, elem_bytes=2):
    """Everything a decode step moves at minimum: the KV read above, the raw
    new q/k/v read, the cache append write and the output write."""
    n = len(cached_lengths)
    per_seq = elem_bytes * head_dim * (n_q_heads + 2 * n_kv_heads + 2 * n_kv_heads + n_q_heads)
    return decode_kv_read_bytes(cached_lengths, n_kv_heads, head_dim, elem_bytes) + n * per_seq


def append_pairs(start_positions, new_lengths):
    """Unmasked (query, key) pairs per query head of an append: new token j of a
    sequence with p cached tokens sees p + j + 1 keys, so n p + n (n + 1) / 2."""
    return sum(int(n) * int(p) + int(n) * (int(n) + 1) // 2 for p, n in zip(start_positions, new_lengths))


def append_flops(start_positions, new_lengths, n_q_heads, head_dim=128):
    """4 d flops per unmasked pair and query head, as for prefill."""
    return 4 * head_dim * n_q_heads * append_pairs(start_positions, new_lengths)
