"""The oracle against library routines, closed forms and invariants (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(name):
    oracle_pins.ALL_PINS[name](None)


def test_sparse_contract_violations_rejected():
    """The oracle refuses a sparse call outside its definition: a causal mask, a count
    outside [0, stride], a counted row outside the pool."""
    import numpy as np

    from oracle import oracle as O

    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 1, 2, 8)).astype(np.float32)
    pool = rng.standard_normal((10, 1, 8)).astype(np.float32)
    idx = rng.integers(0, 10, size=(2, 4)).astype(np.int32)
    ok = dict(scale=0.5, indices=idx, topk_lengths=np.array([4, 2], np.int32))
    O.attention(q, pool, pool, **ok)
    bad_idx = idx.copy()
    bad_idx[1, 1] = 10
    cases = [dict(ok, causal=True), dict(ok, topk_lengths=np.array([5, 2], np.int32)),
             dict(ok, topk_lengths=np.array([4, -1], np.int32)), dict(ok, indices=bad_idx)]
    for kw in cases:
        with pytest.raises(RuntimeError):
            O.attention(q, pool, pool, **kw)
    bad_idx[1, 1] = idx[1, 1]
    bad_idx[1, 2] = -1  # past the count of 2: not part of the call
    bad_idx[1, 3] = 99
    O.attention(q, pool, pool, **dict(ok, indices=bad_idx))


def test_ragged_kv_layout_contract_violations_rejected():
    """The oracle refuses a ragged KV layout whose sequence would read past the cache,
    or that is combined with a page table or a sparse list."""
    import numpy as np

    from oracle import oracle as O

    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 1, 2, 8)).astype(np.float32)
    cache = rng.standard_normal((20, 1, 8)).astype(np.float32)
    lens = np.array([5, 7], np.uint32)
    ok = dict(scale=0.5, valid_length=lens, max_seq_len=8)
    O.attention(q, cache, cache, kv_offsets=np.array([0, 13], np.uint32), **ok)
    with pytest.raises(RuntimeError):  # rows 14 .. 20 of a 20-row cache
        O.attention(q, cache, cache, kv_offsets=np.array([0, 14], np.uint32), **ok)
    with pytest.raises(RuntimeError):  # no valid_length: 8 keys each
        O.attention(q, cache, cache, kv_offsets=np.array([0, 13], np.uint32), scale=0.5,
                    max_seq_len=8)
