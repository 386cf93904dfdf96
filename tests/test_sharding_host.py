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


# ------------------------------------------------------------- model-buffer utilities

@pytest.mark.parametrize("scheme", ["contiguous", "zigzag"])
@pytest.mark.parametrize("seq_dim", [0, 1, 2])
def test_buffer_shards_follow_the_oracle_rows_and_round_trip(scheme, seq_dim):
    import torch
    rng = np.random.default_rng(seq_dim)
    shape = [3, 5, 7]
    shape[seq_dim] = 48
    x = rng.standard_normal(shape).astype(np.float32)
    n = 4
    rows = oracle.shard_rows(48, n, scheme)
    for kind in (np.asarray, torch.from_numpy):
        xs = [sharding.shard_buffer(kind(x), seq_dim, n, r, scheme) for r in range(n)]
        for r in range(n):
            assert np.array_equal(np.asarray(xs[r]), np.take(x, rows[r], axis=seq_dim))
        back = sharding.unshard_buffers(xs, seq_dim, scheme)
        assert np.array_equal(np.asarray(back), x)


def test_labels_shifted_before_sharding_stay_aligned():
    """Every rank's label for a token is the next global token only when the shift comes first."""
    ids = np.arange(64, dtype=np.int64)[None, :] + 1000
    n = 4
    pos = sharding.shard_positions(64, n, "zigzag")
    before = [sharding.shard_buffer(sharding.shift_labels(ids), 1, n, r) for r in range(n)]
    after = [sharding.shift_labels(sharding.shard_buffer(ids, 1, n, r)) for r in range(n)]
    for r in range(n):
        want = np.where(pos[r] + 1 < 64, pos[r] + 1001, -100)
        assert np.array_equal(before[r][0], want)
        assert not np.array_equal(after[r][0], want)      # the misalignment the shift order avoids


def test_maybe_context_parallel_shards_in_place_and_restores():
    import torch
    ids = torch.arange(2 * 32).reshape(2, 32)
    labels = sharding.shift_labels(ids.clone())
    mask = torch.ones(2, 32, dtype=torch.bool)
    orig_ids, orig_mask = ids.clone(), mask.clone()
    pos = sharding.shard_positions(32, 4, "zigzag")[1]
    with sharding.maybe_context_parallel([ids, labels, mask], [1, 1, 1], no_restore_buffers={labels},
                                         n=4, rank=1):
        assert ids.shape == (2, 8) and torch.equal(ids, orig_ids[:, pos])
        assert torch.equal(labels, sharding.shift_labels(orig_ids)[:, pos])
    assert torch.equal(ids, orig_ids) and torch.equal(mask, orig_mask)    # restored
    assert labels.shape == (2, 8)                                          # left sharded, as asked
    # disabled: a no-op on the very same tensors
    before = ids.data_ptr()
    cm = sharding.maybe_context_parallel([ids], [1], n=1)
    with cm:
        assert ids.data_ptr() == before and ids.shape == (2, 32)
    with pytest.raises(RuntimeError):
        with cm:
            pass
