"""Host-side sharding of the product against the oracle's own sharding and closed forms."""
import numpy as np
import pytest

import oracle
from ring_attention_ringattn_amd import sharding


@pytest.mark.parametrize("n", [1, 2, 4, 8])
@pytest.mark.parametrize("scheme", ["contiguous", "zigzag"])
def test_shards_match_oracle(n, scheme):
    s = 32 * n
    mine = sharding.shard_positions(s, n, scheme)
    ref = oracle.shard_rows(s, n, scheme)
    for a, b in zip(mine, ref):
        assert a.dtype == np.int32 and np.array_equal(a, b)


def test_zigzag_closed_form_counts():
    # 131072 tokens over 8 ranks (c = 8192) and 262144 over 8 (c = 16384), per rank and q-head
    for s, n, total in ((131072, 8, 1_073_750_016), (262144, 8, 4_294_983_680), (8192, 4, 8_389_632)):
        c = s // (2 * n)
        for r in range(n):
            assert sum(sharding.causal_pairs_zigzag(n, c, r, j) for j in range(n)) == total
    # and the closed form equals counting with the oracle's mask on small cases
    for n, c in ((2, 4), (4, 3), (8, 2)):
        pos = sharding.shard_positions(2 * n * c, n, "zigzag")
        for r in range(n):
            for j in range(n):
                assert oracle.count_allowed_pairs(pos[r], pos[j], "causal") == \
                    sharding.causal_pairs_zigzag(n, c, r, j)


def test_ring_block_schedule():
    n = 8
    for r in range(n):
        seen = [sharding.block_of(r, t, n) for t in range(n)]
        assert seen[0] == r and sorted(seen) == list(range(n))
        # block at step t+1 is the one the previous rank held at step t
        for t in range(n - 1):
            assert sharding.block_of(r, t + 1, n) == sharding.block_of((r - 1) % n, t, n)
