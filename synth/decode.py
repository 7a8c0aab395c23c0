"""Seeded inputs of the FP8 sparse decode workload (MQA over a paged cache of
656-byte token rows).

Recipe: numpy.random.default_rng(seed); draw order Q, cache values, page
permutation, indices.  Q is N(0,1) rounded to bfloat16.  Every token's 576 key
values are N(0,1); the first 512 are quantised per 1x128 tile with a descale
amax/448 rounded up to a power of two (the reference quantiser of the FlashMLA
FP8 KV-cache article) and E4M3 rounding by torch's CPU cast; the last 64 are
rounded to bfloat16.  Pages: sum_b ceil(Lkv_b/page_size) + 3 spare pages in a
random permutation; block-table entries past a sequence's pages point at a
spare page; slots past Lkv hold `fill` (random bytes, or NaN codes and NaN
descales; drawn from a separate generator).  Indices: for each query token, `topk` distinct positions drawn
uniformly from [0, Lkv_b) (all of them when Lkv_b < topk) in random order, each
written as the cache row that holds it, page * page_size + slot with page =
block_table[b, pos // page_size] and slot = pos % page_size (the encoding of
the FlashMLA FP8 sparse decoding article's quick-reproduce paragraph); with
`ragged`, a random tail of each list is set to -1, and a few entries are
other values that name no row (negative, or at or past num_pages *
page_size).  The block table and sequence lengths only describe how the cache
was filled; the decode itself reads the rows the indices name.  Only random
draws, layout and torch's casts happen here.
"""
from dataclasses import dataclass
from typing import Tuple

import numpy as np
import torch

D_NOPE = 512
D_ROPE = 64
ROW_BYTES = 656


@dataclass
class DecodeConfig:
    name: str
    lkv: Tuple[int, ...]
    s_q: int
    h_q: int
    topk: int
    page_size: int = 64
    ragged: bool = False
    seed: int = 2000
    description: str = ""


DECODE_CONFIGS = {
    "decode_tiny": DecodeConfig("decode_tiny", lkv=(300, 1000), s_q=2, h_q=64, topk=200, ragged=True,
                                seed=2001, description="B=2, Lkv 300/1000, s_q 2, 64 heads, top-k 200 (ragged)"),
    "decode_b128": DecodeConfig("decode_b128", lkv=(4096,) * 128, s_q=2, h_q=128, topk=2048, seed=2002,
                                description="B=128, s_q 2, 128 heads, top-k 2048 of 4096 cached tokens, "
                                            "page 64"),
    "decode_long16k": DecodeConfig("decode_long16k", lkv=(32768,) * 4, s_q=2, h_q=128, topk=16384, seed=2003,
                                   description="B=4, s_q 2, 128 heads, top-k 16384 of 32768 cached tokens, "
                                               "page 64 (few query tokens, long lists: the split-list path)"),
}


@dataclass
class DecodeProblem:
    cfg: DecodeConfig
    q: np.ndarray            # float32 [B, s_q, h_q, 576] (bfloat16 values)
    kv_cache: np.ndarray     # uint8 [num_pages, page_size, 656]
    indices: np.ndarray      # int32 [B, s_q, topk]
    block_table: np.ndarray  # int32 [B, max_pages]
    seqlens_kv: np.ndarray   # int32 [B]
    softmax_scale: float

    def oracle_kwargs(self):
        return dict(q=self.q, kv_cache=self.kv_cache, indices=self.indices,
                    softmax_scale=self.softmax_scale)

    def to_device(self, device="cuda"):
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        return dict(q=t(self.q).to(torch.bfloat16), kv_cache=t(self.kv_cache), indices=t(self.indices))

    def row_of(self, b, pos):
        """Cache row (page * page_size + slot) holding token position pos of
        sequence b."""
        ps = self.kv_cache.shape[1]
        return int(self.block_table[b, pos // ps]) * ps + pos % ps


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _token_rows(rng, n):
    """n cache rows of 656 bytes from N(0,1) keys."""
    x = rng.standard_normal((n, D_NOPE + D_ROPE), dtype=np.float32)
    nope = x[:, :D_NOPE].reshape(n, 4, 128)
    amax = np.abs(nope).max(axis=2)
    m, e = np.frexp(amax.astype(np.float64) / 448.0)
    descale = np.where(m == 0.5, np.ldexp(0.5, e), np.ldexp(1.0, e)).astype(np.float32)
    descale[amax == 0] = 1.0
    codes = torch.from_numpy(np.ascontiguousarray(nope / descale[:, :, None])).clamp(-448, 448) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(n, D_NOPE)
    rope = _bf16(x[:, D_NOPE:]).view(torch.int16).numpy().view(np.uint8).reshape(n, 2 * D_ROPE)
    return np.concatenate([codes, descale.view(np.uint8).reshape(n, 16), rope], axis=1)


def make_decode_problem(cfg, seed=None, fill="random", lkv=None, s_q=None, h_q=None, topk=None,
                        page_size=None, ragged=None):
    if isinstance(cfg, str):
        cfg = DECODE_CONFIGS[cfg]
    over = dict(lkv=lkv, s_q=s_q, h_q=h_q, topk=topk, page_size=page_size, ragged=ragged)
    cfg = DecodeConfig(**{**cfg.__dict__, **{k: v for k, v in over.items() if v is not None}})
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B = len(cfg.lkv)
    ps = cfg.page_size
    q = _bf16(rng.standard_normal((B, cfg.s_q, cfg.h_q, D_NOPE + D_ROPE), dtype=np.float32)).float().numpy()
    n_pages_seq = [-(-l // ps) for l in cfg.lkv]
    total_pages = sum(n_pages_seq) + 3
    rows = _token_rows(rng, total_pages * ps).reshape(total_pages, ps, ROW_BYTES)
    perm = rng.permutation(total_pages)
    max_pages = max(max(n_pages_seq), 1)
    block_table = np.full((B, max_pages), perm[-1], dtype=np.int32)
    kv_cache = np.empty_like(rows)
    if fill == "nan":
        kv_cache[:] = 0x7F
        kv_cache[:, :, D_NOPE:D_NOPE + 16] = np.frombuffer(np.full(4, np.nan, np.float32).tobytes(), np.uint8)
    else:
        # from a generator of its own, so that the fill never changes the other draws
        fill_rng = np.random.default_rng((cfg.seed if seed is None else seed) + 7777)
        kv_cache[:] = fill_rng.integers(0, 256, size=kv_cache.shape, dtype=np.uint8)
    used = 0
    for b in range(B):
        pages = perm[used:used + n_pages_seq[b]]
        block_table[b, :len(pages)] = pages
        for i, pg in enumerate(pages):
            n = min(ps, cfg.lkv[b] - i * ps)
            kv_cache[pg, :n] = rows[used + i, :n]
        used += n_pages_seq[b]
    n_rows = total_pages * ps
    indices = np.full((B, cfg.s_q, cfg.topk), -1, dtype=np.int32)
    for b in range(B):
        for s in range(cfg.s_q):
            take = min(cfg.topk, cfg.lkv[b])
            pos = rng.permutation(cfg.lkv[b])[:take].astype(np.int64)
            sel = (block_table[b, pos // ps].astype(np.int64) * ps + pos % ps).astype(np.int32)
            if cfg.ragged:
                keep = int(rng.integers(take // 2, take + 1))
                sel = sel[:keep]
                bad = np.flatnonzero(rng.random(sel.size) < 0.02)
                # entries that name no row: past the cache, or negative other than -1
                junk = np.where(rng.random(bad.size) < 0.5, n_rows + rng.integers(0, 50, size=bad.size),
                                -2 - rng.integers(0, 1000, size=bad.size))
                sel[bad] = junk
            indices[b, s, :sel.size] = sel
    return DecodeProblem(cfg=cfg, q=q, kv_cache=kv_cache, indices=indices, block_table=block_table,
                         seqlens_kv=np.asarray(cfg.lkv, dtype=np.int32),
                         softmax_scale=float(1.0 / np.sqrt(D_NOPE + D_ROPE)))
