"""fp64 oracle of FP8 sparse decode over a paged 656-byte KV cache.

Test infrastructure only (see the package docstring).  Plain NumPy in float64.

What is computed (the FlashMLA FP8 sparse decoding article: section "FP8
KVCache format" for the cache row, "Quant/dequant source" for dequantisation,
and its MQA description of the decode step):

  * the attention is multi-query: every query head attends to the same single
    KV head; the key has 576 dimensions, the value is the first 512 of them;
  * a cache row (one token) is 656 bytes: 512 E4M3 codes (the first 512 key
    dimensions, in four 1x128 tiles), then 4 float32 descales (one per tile),
    then 64 bfloat16 values (dimensions 512..575, kept unquantised);
  * dequantised key k^ = (code * descale of its tile) for the first 512
    dimensions, the bfloat16 values for the last 64; v^ = k^[:512];
  * for query token (b, s) and head h, the attended set is the list
    indices[b, s, :]; each entry names one cache row as page-block index *
    page_block_size + offset within the block, and -1 marks an unused entry
    (the article's quick-reproduce paragraph: indices of shape (batch,
    seq_len_q, topk) passed as indices_in_kvcache).  So entry e is the row
    kv_cache[e // page_size, e % page_size]; an entry outside
    [0, num_pages * page_size) selects nothing (the plain reading of "-1 is
    invalid", extended to every entry that names no row), and an entry listed
    twice counts twice (each entry is one term of the sum);
  * score_j = softmax_scale * q[b, s, h, :] . k^_j (576 dimensions);
    O = sum_j softmax_j(score) v^_j; LSE = ln sum_j exp(score_j);
  * an empty set gives O = 0 and LSE = -FLT_MAX (the convention of "Quant
    Block Sparse Attention", "Sparse indices & PA page table", for an empty
    sparse task).

Reading where the article leaves a step open: the LSE is laid out
[B, h_q, s_q].  No block table and no sequence length enter the decode: the
index list addresses cache rows directly.
"""
import numpy as np
import torch

from . import e4m3

D_NOPE = 512
D_ROPE = 64
D_K = D_NOPE + D_ROPE
ROW_BYTES = 656
TILE = 128
NEG_FLT_MAX = -3.4028234663852886e38


def dequant_rows(rows):
    """uint8 [..., 656] cache rows -> float64 [..., 576] dequantised keys."""
    rows = np.asarray(rows, dtype=np.uint8)
    codes = rows[..., :D_NOPE]
    scales = np.ascontiguousarray(rows[..., D_NOPE:D_NOPE + 16]).view(np.float32).astype(np.float64)
    rope_bits = np.ascontiguousarray(rows[..., D_NOPE + 16:]).view(np.uint16)
    rope = torch.from_numpy(rope_bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    nope = e4m3.decode(codes) * np.repeat(scales, TILE, axis=-1)
    return np.concatenate([nope, rope], axis=-1)


def gather_rows(kv_cache, entries):
    """Cache rows named by index entries (all valid): entry e is the row at
    page e // page_size, slot e % page_size."""
    page_size = kv_cache.shape[1]
    entries = np.asarray(entries, dtype=np.int64)
    return kv_cache[entries // page_size, entries % page_size].reshape(len(entries), ROW_BYTES)


def valid_entries(idx, kv_cache):
    """The entries of one index list that name a cache row, in list order."""
    idx = np.asarray(idx, dtype=np.int64)
    rows = kv_cache.shape[0] * kv_cache.shape[1]
    return idx[(idx >= 0) & (idx < rows)]


def sparse_decode(q, kv_cache, indices, softmax_scale, with_abs=False):
    """q: float [B, s_q, h_q, 576] (bfloat16 values); kv_cache: uint8
    [num_pages, page_size, 656] (or [num_pages, page_size, 1, 656]);
    indices: int [B, s_q, topk] of cache rows (page * page_size + slot, -1
    unused).  Returns (O float64 [B, s_q, h_q, 512],
    LSE float64 [B, h_q, s_q]); with with_abs, also
    A = sum_j softmax_j |v^_j| (same shape as O), the scale of the error that
    rounding each probability by a relative amount causes in O."""
    q = np.asarray(q, dtype=np.float64)
    kv_cache = np.asarray(kv_cache, dtype=np.uint8)
    kv_cache = kv_cache.reshape(kv_cache.shape[0], kv_cache.shape[1], ROW_BYTES)
    B, s_q, h_q, _ = q.shape
    out = np.zeros((B, s_q, h_q, D_NOPE))
    absw = np.zeros((B, s_q, h_q, D_NOPE))
    lse = np.full((B, h_q, s_q), NEG_FLT_MAX)
    for b in range(B):
        for s in range(s_q):
            idx = valid_entries(indices[b, s], kv_cache)
            if idx.size == 0:
                continue
            k = dequant_rows(gather_rows(kv_cache, idx))                      # [n, 576]
            scores = softmax_scale * (q[b, s] @ k.T)                          # [h, n]
            mx = scores.max(axis=1, keepdims=True)
            w = np.exp(scores - mx)
            l = w.sum(axis=1, keepdims=True)
            out[b, s] = (w @ k[:, :D_NOPE]) / l
            absw[b, s] = (w @ np.abs(k[:, :D_NOPE])) / l
            lse[b, :, s] = (mx + np.log(l))[:, 0]
    return (out, lse, absw) if with_abs else (out, lse)
