"""Oracle of the scheduling pre-pass: task costs and the task order.

Test infrastructure only (see the package docstring).  Plain Python/NumPy.

"Quant Block Sparse Attention" ("Sparse indices & PA page table") has a
metadata operator read the sparse workload on the device and split the
(batch, query head, query block) tasks between cores before the attention
runs.  The order defined here is the plain reading for a GPU whose dispatcher
hands out tasks as cores free up:

  * task id of (sequence b, q-head h, Q tile m) = (b * Hq + h) * Mt + m, with
    Mt = ceil(max_seqlen_q / 128);
  * cost of a task = the number of its selected KV tiles that hold at least one
    key some query of the Q tile may attend to (key below Lkv and, in causal
    mode, at or below the query's bottom-right position), 0 for a Q tile that
    starts at or beyond Lq;
  * the GPU hands workgroup i to XCD i mod 8 (eight XCDs, each with its own
    L2), so position i of the order runs on XCD i mod 8.  When Hq is a multiple
    of 8, XCD x is given the contiguous q-head range [x*Hq/8, (x+1)*Hq/8) (all
    its sequences and Q tiles, so the eight shares have the same shape and the
    K/V of a kv-head stays within one or two XCDs); its tasks are sorted by
    decreasing min(cost, 1023), equal values by increasing id, and its j-th
    task takes position 8j + x.  Otherwise all tasks form one list, sorted the
    same way, and the j-th task takes position j.

The selection of KV tiles is the one of the attention oracle: mask bytes
(tiles beyond the mask width are off), or the valid entries of an index list,
or every tile when neither is given.
"""
import numpy as np

TILE = 128
COST_CAP = 1023


def _ceil_div(a, b):
    return -(-a // b)


def _selected(block_mask, index_form, b, h, m, n_tiles):
    """Boolean [n_tiles]: KV tiles the sparsity argument selects for Q tile m."""
    sel = np.zeros(n_tiles, dtype=bool)
    if index_form is not None:
        sparse_indices, sparse_seq_len = index_form
        length = max(int(sparse_seq_len[b, h, m]), 0)
        for e in np.asarray(sparse_indices[b, h, m, :length]):
            if 0 <= e < n_tiles:
                sel[e] = True
    elif block_mask is None:
        sel[:] = True
    else:
        row = np.asarray(block_mask[b, h, m, :n_tiles]) != 0
        sel[:row.size] = row
    return sel


def task_costs(cu_seqlens_q, seqlens_kv, num_heads_q, max_seqlen_q, causal=True,
               block_mask=None, sparse_indices=None, sparse_seq_len=None):
    """int64 [B * Hq * Mt] cost of every task, by task id."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lkv_all = np.asarray(seqlens_kv, dtype=np.int64)
    B = lkv_all.size
    mt = _ceil_div(int(max_seqlen_q), TILE)
    index_form = None if sparse_indices is None else (sparse_indices, sparse_seq_len)
    cost = np.zeros(B * num_heads_q * mt, dtype=np.int64)
    for b in range(B):
        lq = int(cu[b + 1] - cu[b])
        lkv = int(lkv_all[b])
        n_tiles = _ceil_div(lkv, TILE)
        for h in range(num_heads_q):
            for m in range(mt):
                if m * TILE >= lq:
                    continue
                last_query = min(m * TILE + TILE, lq) - 1
                reach = lkv - lq + last_query if causal else lkv - 1   # largest visible key
                sel = _selected(block_mask, index_form, b, h, m, n_tiles)
                tiles = np.nonzero(sel)[0]
                # a tile holds a visible key iff its first key is <= reach (and < lkv)
                cost[(b * num_heads_q + h) * mt + m] = int(np.sum(tiles * TILE <= reach))
    return cost


XCDS = 8


def schedule(costs, num_heads_q, max_seqlen_q):
    """Task id at every launch position (see the module docstring)."""
    c = np.minimum(np.asarray(costs, dtype=np.int64), COST_CAP)
    n = c.size
    ids = np.arange(n)
    if num_heads_q % XCDS != 0:
        return np.lexsort((ids, -c)).astype(np.int32)
    mt = _ceil_div(int(max_seqlen_q), TILE)
    head = (ids // mt) % num_heads_q
    share = head // (num_heads_q // XCDS)             # the XCD that owns the head
    order = np.lexsort((ids, -c, share))              # share-major, then cost, then id
    per = n // XCDS
    out = np.empty(n, dtype=np.int32)
    j = np.arange(n)
    out[(j % per) * XCDS + j // per] = order          # j-th task of share x -> 8j + x
    return out
