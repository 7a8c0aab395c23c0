"""Pins of the scheduling oracle (oracle/schedule.py): task costs against a
brute-force count over individual queries and keys, hand-worked examples, and
the ordering rule."""
import numpy as np
import pytest

from oracle import schedule as S

TILE = 128


def brute_costs(cu, lkv, hq, max_lq, causal, mask=None, idx=None, slen=None):
    """Cost by definition: selected KV tiles with at least one (query, key) pair
    of the Q tile that attention may use, counted key by key."""
    B = len(lkv)
    mt = -(-max_lq // TILE)
    out = np.zeros(B * hq * mt, dtype=np.int64)
    for b in range(B):
        lq = cu[b + 1] - cu[b]
        n_tiles = -(-lkv[b] // TILE)
        for h in range(hq):
            for m in range(mt):
                queries = range(m * TILE, min(m * TILE + TILE, lq))
                if idx is not None:
                    listed = {int(e) for e in idx[b, h, m, :max(int(slen[b, h, m]), 0)]}
                count = 0
                for n in range(n_tiles):
                    if idx is not None:
                        if n not in listed:
                            continue
                    elif mask is not None:
                        if n >= mask.shape[3] or mask[b, h, m, n] == 0:
                            continue
                    usable = False
                    for t in queries:
                        pos = lkv[b] - lq + t
                        for j in range(n * TILE, min(n * TILE + TILE, lkv[b])):
                            if not causal or j <= pos:
                                usable = True
                                break
                        if usable:
                            break
                    count += usable
                out[(b * hq + h) * mt + m] = count
    return out


def random_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    lq = rng.integers(1, 400, size=B)
    lkv = lq + rng.integers(0, 300, size=B)
    hq = int(rng.integers(1, 4))
    max_lq = int(lq.max()) + int(rng.integers(0, 200))
    mt = -(-max_lq // TILE)
    kb = int(rng.integers(1, 7))
    cu = np.concatenate([[0], np.cumsum(lq)])
    mask = (rng.random((B, hq, mt, kb)) < 0.6).astype(np.uint8)
    idx = np.zeros((B, hq, mt, kb + 2), dtype=np.int32)
    for b in range(B):          # ids in -2 .. kb+2, no repeats within a row
        for h in range(hq):
            for m in range(mt):
                idx[b, h, m] = rng.permutation(np.arange(-2, kb + 3))[:kb + 2]
    slen = rng.integers(-1, kb + 5, size=(B, hq, mt)).astype(np.int32)   # may exceed the row
    return cu, lkv, hq, max_lq, mask, idx, slen


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [True, False])
def test_costs_match_brute_force(seed, causal):
    cu, lkv, hq, max_lq, mask, idx, slen = random_case(seed)
    for form in ("dense", "mask", "list"):
        kw = {}
        if form == "mask":
            kw = dict(block_mask=mask)
        elif form == "list":
            kw = dict(sparse_indices=idx, sparse_seq_len=slen)
        got = S.task_costs(cu, lkv, hq, max_lq, causal, **kw)
        want = brute_costs(cu, lkv, hq, max_lq, causal,
                           mask=mask if form == "mask" else None,
                           idx=idx if form == "list" else None,
                           slen=slen if form == "list" else None)
        np.testing.assert_array_equal(got, want, err_msg=form)


# Hand-worked: B=1, Hq=2, three Q tiles and three KV tiles, causal.
HAND_MASK = np.array([[[[1, 1, 1], [0, 1, 1], [1, 0, 1]],
                       [[0, 1, 1], [1, 1, 0], [1, 1, 1]]]], dtype=np.uint8)


def test_hand_example_aligned():
    # Lq = Lkv = 384: Q tile m reaches KV tile m.
    # h0: m0 {0} -> 1, m1 {1} -> 1, m2 {0,2} -> 2; h1: m0 {} -> 0, m1 {0,1} -> 2, m2 {0,1,2} -> 3
    c = S.task_costs([0, 384], [384], 2, 384, True, block_mask=HAND_MASK)
    np.testing.assert_array_equal(c, [1, 1, 2, 0, 2, 3])
    np.testing.assert_array_equal(S.schedule(c, 2, 384), [5, 2, 4, 0, 1, 3])


def test_hand_example_offset():
    # Lq = 300, Lkv = 384: queries sit at positions 84..383, so Q tile 0 reaches
    # key 211 (KV tile 1) and Q tiles 1 and 2 reach KV tile 2.
    c = S.task_costs([0, 300], [384], 2, 300, True, block_mask=HAND_MASK)
    np.testing.assert_array_equal(c, [2, 2, 2, 1, 2, 3])
    np.testing.assert_array_equal(S.schedule(c, 2, 300), [5, 0, 1, 2, 4, 3])


def test_hand_example_non_causal_and_beyond_lq():
    # Two sequences, max_seqlen_q 300 -> 3 Q tiles each; sequence 1 has
    # Lq = 100, so its Q tiles 1 and 2 cost 0.  Non-causal: every selected tile
    # below Lkv counts.
    mask = np.concatenate([HAND_MASK, HAND_MASK[:, ::-1]], axis=0)
    c = S.task_costs([0, 300, 400], [384, 200], 2, 300, False, block_mask=mask)
    # b0: rows as in the mask (3 KV tiles): 3,2,2 | 2,2,3 ; b1 (2 KV tiles, h order
    # swapped): h0 = HAND_MASK h1 rows: m0 [0,1] -> 1; h1 = HAND_MASK h0: m0 [1,1] -> 2
    np.testing.assert_array_equal(c, [3, 2, 2, 2, 2, 3, 1, 0, 0, 2, 0, 0])
    np.testing.assert_array_equal(S.schedule(c, 2, 300), [0, 5, 1, 2, 3, 4, 9, 6, 7, 8, 10, 11])


def test_index_list_hand_example():
    # Lists with junk (-1, past the KV length), an unsorted order, and an
    # invalid tail beyond sparse_seq_len; Lq = Lkv = 384.
    idx = np.array([[[[2, -1, 0, 7], [9, 1, 0, 0], [2, 0, 5, 1]],
                     [[1, 2, -3, 0], [0, 0, 0, 0], [1, 2, 0, -1]]]], dtype=np.int32)
    slen = np.array([[[3, 2, 2], [2, 0, 3]]], dtype=np.int32)
    c = S.task_costs([0, 384], [384], 2, 384, True, sparse_indices=idx, sparse_seq_len=slen)
    # h0: m0 {2,0} -> tile 0 -> 1; m1 {1} -> 1; m2 {2,0} -> 2
    # h1: m0 {1,2} -> 0; m1 {} -> 0; m2 {1,2,0} -> 3
    np.testing.assert_array_equal(c, [1, 1, 2, 0, 0, 3])
    np.testing.assert_array_equal(S.schedule(c, 2, 384), [5, 2, 0, 1, 3, 4])


def test_dense_costs_closed_form():
    # No sparsity argument, Lq = Lkv = 128 * k, causal: Q tile m costs m + 1.
    c = S.task_costs([0, 640], [640], 1, 640, True)
    np.testing.assert_array_equal(c, [1, 2, 3, 4, 5])
    np.testing.assert_array_equal(S.schedule(c, 1, 640), [4, 3, 2, 1, 0])


def test_order_rule_and_cap():
    c = np.array([5, 2000, 1023, 0, 1500, 5, 7])
    s = S.schedule(c, 7, 128)          # 7 heads, one Q tile each: a single list
    np.testing.assert_array_equal(s, [1, 2, 4, 6, 0, 5, 3])
    assert s.dtype == np.int32


@pytest.mark.parametrize("seed", range(4))
def test_schedule_is_sorted_permutation(seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1100, size=3000)
    s = S.schedule(c, 3, 128 * 1000)   # 3 heads: a single list
    assert sorted(s.tolist()) == list(range(c.size))
    key = np.minimum(c[s], 1023)
    assert np.all(np.diff(key) <= 0)
    ties = np.diff(key) == 0
    assert np.all(np.diff(s)[ties] > 0)


def test_reach_on_a_tile_boundary():
    # Lq = 256, Lkv = 257: the last query of Q tile 0 sits at position 128, the
    # first key of KV tile 1, so that tile counts; Q tile 1 reaches key 256, the
    # only key of KV tile 2.
    c = S.task_costs([0, 256], [257], 1, 256, True)
    np.testing.assert_array_equal(c, [2, 3])
    # one key short of the boundary: Lkv = 256 puts the last query at 127
    c = S.task_costs([0, 256], [256], 1, 256, True)
    np.testing.assert_array_equal(c, [1, 2])


def test_xcd_shares_hand_example():
    # Hq = 8, one sequence of 2 Q tiles: task id = 2h + m; head h belongs to
    # XCD h.  Costs (h, m) and the order they give: h0 (1, 3) [1, 0];
    # h1 (2, 2) [2, 3] (tie: ids); h2 (0, 5) [5, 4]; h3 (1, 4) [7, 6];
    # h4 (2, 2) [8, 9]; h5 (9, 9) [10, 11]; h6 (0, 0) [12, 13]; h7 (7, 8) [15, 14].
    # Position 8j + x holds the j-th task of XCD x.
    c = np.array([1, 3, 2, 2, 0, 5, 1, 4, 2, 2, 9, 9, 0, 0, 7, 8])
    s = S.schedule(c, 8, 256)
    want = np.array([1, 2, 5, 7, 8, 10, 12, 15,      # j = 0 for x = 0..7
                     0, 3, 4, 6, 9, 11, 13, 14])     # j = 1
    np.testing.assert_array_equal(s, want)


@pytest.mark.parametrize("seed", range(3))
def test_xcd_shares_properties(seed):
    rng = np.random.default_rng(seed)
    hq, mt, B = 16, 7, 3
    c = rng.integers(0, 1100, size=B * hq * mt)
    s = S.schedule(c, hq, mt * 128)
    assert sorted(s.tolist()) == list(range(c.size))
    head = (s // mt) % hq
    for x in range(8):
        mine = s[x::8]                                      # what XCD x runs, in order
        assert set(head[x::8].tolist()) == {2 * x, 2 * x + 1}
        key = np.minimum(c[mine], 1023)
        assert np.all(np.diff(key) <= 0)
        assert np.all(np.diff(mine)[np.diff(key) == 0] > 0)
