"""Pins of the FP8 sparse decode oracle (oracle/decode.py): a hand-built cache
row, hand-built index entries (page-block index * page_block_size + offset,
-1 unused: the FlashMLA FP8 sparse decoding article, quick-reproduce
paragraph), a scalar brute force, closed forms, the handling of invalid and
repeated indices, invariances, and dense attention against torch."""
import math
import struct

import numpy as np
import pytest
import torch

from oracle import decode as D
from oracle import e4m3
from synth import make_decode_problem


def test_hand_built_row():
    # codes from the E4M3 format: 0x7E = 448, 0x38 = 1.0 (0 0111 000),
    # 0xB8 = -1.0, 0x01 = 2^-9; descales 0.25, 1, 2^-10, 8; bfloat16 RoPE
    # 0x3F80 = 1.0, 0xC000 = -2.0
    row = np.zeros(656, dtype=np.uint8)
    row[0], row[1], row[128], row[256], row[384] = 0x7E, 0x38, 0xB8, 0x01, 0x38
    row[512:528] = np.frombuffer(struct.pack("<4f", 0.25, 1.0, 2.0 ** -10, 8.0), dtype=np.uint8)
    row[528:530] = [0x80, 0x3F]
    row[530:532] = [0x00, 0xC0]
    k = D.dequant_rows(row[None])[0]
    assert k.shape == (576,)
    assert k[0] == 112.0 and k[1] == 0.25 and k[128] == -1.0
    assert k[256] == 2.0 ** -19 and k[384] == 8.0
    assert k[512] == 1.0 and k[513] == -2.0
    assert np.count_nonzero(k) == 7


def _marked_cache(num_pages, page_size):
    """A cache whose row (page g, slot t) has code 1.0 at dimension 0, zeros
    elsewhere and descale 1 + g * page_size + t on its first tile, so a decode
    over one entry returns that number at output dimension 0."""
    cache = np.zeros((num_pages, page_size, 656), dtype=np.uint8)
    for g in range(num_pages):
        for t in range(page_size):
            cache[g, t, 0] = 0x38                                   # E4M3 1.0
            cache[g, t, 512:528] = np.frombuffer(
                struct.pack("<4f", 1.0 + g * page_size + t, 1.0, 1.0, 1.0), dtype=np.uint8)
    return cache


def test_hand_built_index_entries():
    """Entry e names the row at page e // page_size, slot e % page_size: the
    row of physical page 2, slot 5 of a 32-slot cache is entry 2 * 32 + 5 = 69."""
    cache = _marked_cache(num_pages=3, page_size=32)
    q = np.zeros((1, 5, 2, 576))
    idx = np.full((1, 5, 4), -1, dtype=np.int32)
    idx[0, 0, 2] = 69                     # page 2, slot 5
    idx[0, 1, 0] = 0                      # page 0, slot 0
    idx[0, 2, 3] = 95                     # the last row: page 2, slot 31
    idx[0, 3, :] = [96, -2, 1000, -1]     # past the cache, negative: no row
    idx[0, 4, :2] = [37, 37]              # page 1, slot 5, listed twice
    o, lse = D.sparse_decode(q, cache, idx, softmax_scale=0.1)
    assert o[0, 0, 0, 0] == 1.0 + 2 * 32 + 5 and np.count_nonzero(o[0, 0]) == 2
    assert o[0, 1, 0, 0] == 1.0
    assert o[0, 2, 0, 0] == 1.0 + 2 * 32 + 31
    assert np.all(o[0, 3] == 0) and np.all(lse[0, :, 3] == D.NEG_FLT_MAX)
    assert o[0, 4, 0, 0] == 1.0 + 32 + 5 and lse[0, 0, 4] == math.log(2.0)
    assert np.all(lse[0, :, :3] == 0.0)   # one entry, zero query: ln 1
    # the same entry read with the page size as 64 names another row
    cache64 = _marked_cache(num_pages=2, page_size=64)
    o64, _ = D.sparse_decode(q[:, :1], cache64, idx[:, :1], softmax_scale=0.1)
    assert o64[0, 0, 0, 0] == 1.0 + 69


def scalar_dequant(row):
    scales = struct.unpack("<4f", bytes(row[512:528]))
    out = []
    for i in range(512):
        out.append(float(e4m3.DECODE_TABLE[row[i]]) * scales[i // 128])
    for i in range(64):
        bits = int(row[528 + 2 * i]) | (int(row[529 + 2 * i]) << 8)
        out.append(struct.unpack("<f", struct.pack("<I", bits << 16))[0])
    return out


def test_brute_force_tiny():
    p = make_decode_problem("decode_tiny", lkv=(40, 70), s_q=2, h_q=3, topk=9, ragged=True, seed=5)
    o, lse = D.sparse_decode(**p.oracle_kwargs())
    ps = p.kv_cache.shape[1]
    for b in range(2):
        for s in range(2):
            for h in range(3):
                terms = []
                for j in p.indices[b, s]:
                    if not 0 <= j < p.kv_cache.shape[0] * ps:
                        continue
                    row = p.kv_cache[j // ps, j % ps]
                    k = scalar_dequant(row)
                    sc = p.softmax_scale * sum(float(p.q[b, s, h, d]) * k[d] for d in range(576))
                    terms.append((sc, k[:512]))
                if not terms:
                    assert np.all(o[b, s, h] == 0) and lse[b, h, s] == D.NEG_FLT_MAX
                    continue
                m = max(t[0] for t in terms)
                w = [math.exp(t[0] - m) for t in terms]
                l = sum(w)
                ref = [sum(wi * t[1][d] for wi, t in zip(w, terms)) / l for d in range(512)]
                np.testing.assert_allclose(o[b, s, h], ref, rtol=1e-12, atol=1e-12)
                assert abs(lse[b, h, s] - (m + math.log(l))) < 1e-12


def test_zero_query_closed_form():
    p = make_decode_problem("decode_tiny", seed=6)
    p.q[:] = 0
    o, lse = D.sparse_decode(**p.oracle_kwargs())
    for b in range(2):
        for s in range(2):
            idx = p.indices[b, s]
            idx = idx[(idx >= 0) & (idx < p.kv_cache.shape[0] * p.kv_cache.shape[1])]
            k = D.dequant_rows(D.gather_rows(p.kv_cache, idx))
            np.testing.assert_allclose(o[b, s], np.broadcast_to(k[:, :512].mean(axis=0), o[b, s].shape),
                                       rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, s], math.log(idx.size), rtol=1e-12)


def test_single_entry_and_empty():
    p = make_decode_problem("decode_tiny", seed=7)
    p.indices[:] = -1
    p.indices[0, 0, 5] = p.row_of(0, 17)
    p.indices[1, 1, 0] = p.kv_cache.shape[0] * p.kv_cache.shape[1]   # past the cache: no row
    o, lse = D.sparse_decode(**p.oracle_kwargs())
    k = D.dequant_rows(D.gather_rows(p.kv_cache, np.array([p.row_of(0, 17)])))[0]
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(k[:512], o[0, 0].shape), rtol=1e-14)
    np.testing.assert_allclose(lse[0, :, 0], p.softmax_scale * (p.q[0, 0].astype(np.float64) @ k), rtol=1e-12)
    for b, s in ((0, 1), (1, 0), (1, 1)):
        assert np.all(o[b, s] == 0) and np.all(lse[b, :, s] == D.NEG_FLT_MAX)


def test_order_and_invalid_entries_do_not_matter():
    p = make_decode_problem("decode_tiny", seed=8)
    o1, l1 = D.sparse_decode(**p.oracle_kwargs())
    rng = np.random.default_rng(0)
    idx = p.indices.copy()
    for b in range(2):
        for s in range(2):
            idx[b, s] = rng.permutation(idx[b, s])
    p.indices = idx
    o2, l2 = D.sparse_decode(**p.oracle_kwargs())
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-12)


def test_repeated_entry_equals_a_copied_token():
    """Listing token j twice equals listing j and an identical copy of it."""
    p = make_decode_problem("decode_tiny", lkv=(130, 70), seed=9, ragged=False, topk=20)
    ps = p.kv_cache.shape[1]
    j, spare = int(p.indices[0, 0, 0]), p.row_of(0, 129)   # position 129 holds a copy of row j
    src = p.kv_cache[j // ps, j % ps].copy()
    p.indices[0, 0] = np.where(p.indices[0, 0] == spare, -1, p.indices[0, 0])
    q = make_decode_problem("decode_tiny", lkv=(130, 70), seed=9, ragged=False, topk=20)
    q.indices = p.indices.copy()
    p.indices[0, 0, -1] = j
    q.kv_cache[spare // ps, spare % ps] = src
    q.indices[0, 0, -1] = spare
    o1, l1 = D.sparse_decode(**p.oracle_kwargs())
    o2, l2 = D.sparse_decode(**q.oracle_kwargs())
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_unselected_rows_never_matter():
    a = make_decode_problem("decode_tiny", seed=10, fill="random")
    b = make_decode_problem("decode_tiny", seed=10, fill="nan")
    np.testing.assert_array_equal(a.indices, b.indices)
    oa, la = D.sparse_decode(**a.oracle_kwargs())
    ob, lb = D.sparse_decode(**b.oracle_kwargs())
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_dense_selection_matches_torch_attention():
    p = make_decode_problem("decode_tiny", lkv=(150, 90), s_q=1, h_q=4, topk=150, seed=11)
    for b in range(2):                                  # every token, in order
        p.indices[b, 0] = -1
        p.indices[b, 0, :p.seqlens_kv[b]] = [p.row_of(b, j) for j in range(p.seqlens_kv[b])]
    o, lse = D.sparse_decode(**p.oracle_kwargs())
    for b in range(2):
        n = int(p.seqlens_kv[b])
        rows = np.array([p.row_of(b, j) for j in range(n)])
        k = torch.from_numpy(D.dequant_rows(D.gather_rows(p.kv_cache, rows)))
        q = torch.from_numpy(p.q[b, 0].astype(np.float64))                     # [h, 576]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :], k[None].expand(4, n, 576), k[None, :, :512].expand(4, n, 512),
            scale=p.softmax_scale)[:, 0]
        np.testing.assert_allclose(o[b, 0], ref.numpy(), rtol=1e-10, atol=1e-12)
        ref_lse = torch.logsumexp(p.softmax_scale * (q @ k.T), dim=1)
        np.testing.assert_allclose(lse[b, :, 0], ref_lse.numpy(), rtol=1e-12)


def test_abs_weighted_output():
    """A = sum softmax |v| bounds |O| and equals |O| when all values agree in sign."""
    p = make_decode_problem("decode_tiny", seed=12)
    o, lse, a = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    assert np.all(a >= np.abs(o) - 1e-12)
    ps = p.kv_cache.shape[1]
    for b in range(2):                 # make every value positive: A equals O
        for j in range(p.seqlens_kv[b]):
            r = p.row_of(b, j)
            row = p.kv_cache[r // ps, r % ps]
            row[:512] &= 0x7F            # clear the sign of every code (descales are positive)
    o, lse, a = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    np.testing.assert_allclose(a, o, rtol=1e-12, atol=0)
