"""Algorithmic work counts used for throughput figures, checked by brute force."""

from attention_qk_norm_amd import accounting as A


def brute_pairs(p, n):
    # new token j (position p + j) sees keys 0 .. p + j
    return sum(1 for j in range(n) for key in range(p + n) if key <= p + j)


def test_prefill_pairs_brute_force():
    for lengths in ([1], [5, 0, 3], [64, 65, 7]):
        assert A.prefill_pairs(lengths) == sum(brute_pairs(0, L) for L in lengths)


def test_append_pairs_brute_force_and_chunking():
    assert A.append_pairs([0, 3, 10], [4, 1, 7]) == brute_pairs(0, 4) + brute_pairs(3, 1) + brute_pairs(10, 7)
    # a prompt appended in chunks does exactly the work of one prefill
    L, cuts = 300, [0, 2, 5, 6, 70, 71, 300]
    assert sum(A.append_pairs([a], [b - a]) for a, b in zip(cuts, cuts[1:])) == A.prefill_pairs([L])
    assert A.append_flops([3584] * 4, [512] * 4, 32) == 4 * 128 * 32 * 4 * (512 * 3584 + 512 * 513 // 2)


def test_decode_bytes():
    # one token per sequence: K and V of the cached tokens plus the new one
    assert A.decode_kv_read_bytes([0, 9], 8) == (1 + 10) * 2 * 8 * 128 * 2
    assert A.kv_bytes_per_token(8, layers=36) == 144 * 1024
