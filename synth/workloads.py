"""Workload recipes and the seeded generator.

Recipe (the same for every configuration):
  * numpy.random.default_rng(seed); draw order Q, K, V, mask, page permutation.
  * Q, K, V values are N(0, 1) float32.  They are quantised to E4M3 with a
    descale of amax/448 over each scale group (no power-of-two rounding); the
    E4M3 rounding itself is torch's CPU cast to float8_e4m3fn after clamping
    to +-448.  Scale groups: Q per (token, head); K per tensor (quant 0) or per
    (token, kv-head) (quant 1); V per tensor (quant 0) or per kv-head (quant 1).
  * Paging: num_pages = sum_b ceil(Lkv_b / page_size) + 7 spare pages; the
    physical pages are a random permutation; block_table entries past a
    sequence's last page point at a spare page.  Unused slots (and spare pages)
    hold `fill` (0 for benchmarks, NaN for invariance tests).
  * Block mask [B, Hq, Mt, Kb]: every byte is Bernoulli(keep); for each valid Q
    tile the diagonal band (every KV tile holding a causal position of one of
    its queries) is forced on, plus `window` tiles before it; configurations
    may then force specific rows to zero.  Bits above the causal range, beyond
    Lkv or on Q tiles beyond Lq are left random on purpose (they must have no
    effect).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

TILE = 128
HEAD_DIM = 128
FP8_MAX = 448.0
NAN_CODE = 0x7F   # E4M3FN NaN


@dataclass
class WorkloadConfig:
    name: str
    lq: Tuple[int, ...]
    lkv: Tuple[int, ...]
    hq: int
    hkv: int
    quant_type: int
    kv_layout: int          # 0 NHD, 1 HND
    page_size: int
    keep: float             # Bernoulli keep probability of a non-forced tile (1 - skip_ratio)
    window: int = 0         # extra tiles before the band forced on
    all_ones: bool = False  # mask is literally all ones
    zero_rows: Tuple[Tuple[int, int, int], ...] = ()   # (b, h, m) rows forced all-zero
    causal: bool = True
    seed: int = 1000
    description: str = ""


CONFIGS = {
    "tiny": WorkloadConfig(
        name="tiny", lq=(512,), lkv=(512,), hq=2, hkv=1, quant_type=0, kv_layout=0,
        page_size=64, keep=0.5, seed=1001,
        description="B=1, Lq=Lkv=512, Hq=2, Hkv=1; quant 0, NHD, page 64; skip 0.5"),
    "dense8k": WorkloadConfig(
        name="dense8k", lq=(8192,), lkv=(8192,), hq=32, hkv=8, quant_type=0, kv_layout=0,
        page_size=64, keep=1.0, all_ones=True, seed=1002,
        description="B=1, 8192 tokens, Hq=32, Hkv=8; quant 0, NHD, page 64; all-ones causal mask"),
    "sparse16k": WorkloadConfig(
        name="sparse16k", lq=(16384,), lkv=(16384,), hq=32, hkv=8, quant_type=1, kv_layout=1,
        page_size=32, keep=0.5, seed=1003,
        description="B=1, 16384 tokens, Hq=32, Hkv=8; quant 1, HND, page 32; skip 0.5"),
    "varlen": WorkloadConfig(
        name="varlen", lq=(1024, 2048, 4096, 4096), lkv=(4051, 8115, 12188, 32765), hq=64, hkv=8,
        quant_type=0, kv_layout=0, page_size=64, keep=0.25, zero_rows=((3, 5, 17),), seed=1004,
        description="B=4 chunked prefill, Lkv 4051/8115/12188/32765, Lq 1K/2K/4K/4K tail-aligned, "
                    "Hq=64, Hkv=8; quant 0, NHD, page 64; skip 0.75; row (3,5,17) all zero"),
    "long128k": WorkloadConfig(
        name="long128k", lq=(131072,), lkv=(131072,), hq=32, hkv=4, quant_type=1, kv_layout=0,
        page_size=64, keep=0.1, window=8, seed=1005,
        description="B=1, 131072 tokens, Hq=32, Hkv=4; quant 1, NHD, page 64; band + 8 tiles, "
                    "rest Bernoulli(0.1)"),
}


@dataclass
class Problem:
    """One generated input set (NumPy arrays, uint8 = E4M3 codes)."""
    cfg: WorkloadConfig
    q: np.ndarray
    kcache: np.ndarray
    vcache: np.ndarray
    qscale: np.ndarray
    kscale: np.ndarray
    vscale: np.ndarray
    cu_seqlens_q: np.ndarray
    block_table: np.ndarray
    seqlens_kv: np.ndarray
    block_mask: Optional[np.ndarray]
    max_seqlen_q: int
    softmax_scale: float
    extras: dict = field(default_factory=dict)

    @property
    def quant_type(self):
        return self.cfg.quant_type

    @property
    def page_size(self):
        return self.cfg.page_size

    @property
    def kv_layout(self):
        return self.cfg.kv_layout

    @property
    def causal(self):
        return self.cfg.causal

    def oracle_kwargs(self):
        return dict(q=self.q, kcache=self.kcache, vcache=self.vcache, qscale=self.qscale,
                    kscale=self.kscale, vscale=self.vscale, cu_seqlens_q=self.cu_seqlens_q,
                    block_table=self.block_table, seqlens_kv=self.seqlens_kv,
                    block_mask=self.block_mask, quant_type=self.quant_type,
                    page_size=self.page_size, kv_layout=self.kv_layout,
                    softmax_scale=self.softmax_scale, causal=self.causal)

    def to_device(self, device="cuda"):
        """Torch tensors of every input on `device` (dict, same keys as the C call)."""
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        d = dict(q=t(self.q).view(torch.float8_e4m3fn), kcache=t(self.kcache).view(torch.float8_e4m3fn),
                 vcache=t(self.vcache).view(torch.float8_e4m3fn), qscale=t(self.qscale),
                 kscale=t(self.kscale), vscale=t(self.vscale), cu_seqlens_q=t(self.cu_seqlens_q),
                 block_table=t(self.block_table), seqlens_kv=t(self.seqlens_kv),
                 block_mask=None if self.block_mask is None else t(self.block_mask))
        return d

    @property
    def num_q_tiles(self):
        lq = np.diff(self.cu_seqlens_q)
        return int(((lq + TILE - 1) // TILE).sum()) * self.q.shape[1]


def _quantise(x, descale):
    """x / descale rounded to E4M3 codes by torch's CPU cast (library primitive)."""
    y = torch.from_numpy(np.ascontiguousarray(x / descale))
    return y.clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _descale(amax):
    amax = np.asarray(amax, dtype=np.float32)
    return np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)


def make_problem(cfg, seed=None, fill="zero", lq=None, lkv=None, hq=None, hkv=None,
                 quant_type=None, kv_layout=None, page_size=None, keep=None, mask=True,
                 spare_pages=7, identity_pages=False):
    """Generate one problem.  Keyword overrides replace the matching fields of `cfg`.

    fill: "zero" or "nan" -- contents of unused cache slots, spare pages and
    their K descales (quant 1).
    mask: False gives block_mask=None (the dense path).
    identity_pages: physical page = logical order (no shuffle) -- for invariance tests.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    over = {k: v for k, v in dict(lq=lq, lkv=lkv, hq=hq, hkv=hkv, quant_type=quant_type,
                                   kv_layout=kv_layout, page_size=page_size, keep=keep).items()
            if v is not None}
    if over:
        cfg = WorkloadConfig(**{**cfg.__dict__, **over})
    lq = np.asarray(cfg.lq, dtype=np.int64)
    lkv = np.asarray(cfg.lkv, dtype=np.int64)
    assert lq.shape == lkv.shape
    B, Hq, Hkv, PS = len(lq), cfg.hq, cfg.hkv, cfg.page_size
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T = int(lq.sum())
    total_kv = int(lkv.sum())

    # --- Q -----------------------------------------------------------------
    qf = rng.standard_normal((T, Hq, HEAD_DIM), dtype=np.float32)
    qscale = _descale(np.abs(qf).max(axis=2))
    q = _quantise(qf, qscale[:, :, None])
    del qf
    # --- K -----------------------------------------------------------------
    kf = rng.standard_normal((total_kv, Hkv, HEAD_DIM), dtype=np.float32)
    if cfg.quant_type == 0:
        ks_tok = np.broadcast_to(_descale(np.abs(kf).max()), (total_kv, Hkv))
    else:
        ks_tok = _descale(np.abs(kf).max(axis=2))
    kq = _quantise(kf, ks_tok[:, :, None])
    del kf
    # --- V -----------------------------------------------------------------
    vf = rng.standard_normal((total_kv, Hkv, HEAD_DIM), dtype=np.float32)
    if cfg.quant_type == 0:
        vscale = _descale(np.abs(vf).max()).reshape(1)
        vq = _quantise(vf, vscale[0])
    else:
        vscale = _descale(np.abs(vf).max(axis=(0, 2)))
        vq = _quantise(vf, vscale[None, :, None])
    del vf
    # --- block mask ----------------------------------------------------------
    Mt = int((lq.max() + TILE - 1) // TILE)
    Kb = int((lkv.max() + TILE - 1) // TILE)
    u = rng.random((B, Hq, Mt, Kb), dtype=np.float32)
    if cfg.all_ones:
        bm = np.ones((B, Hq, Mt, Kb), dtype=np.uint8)
    else:
        bm = (u < cfg.keep).astype(np.uint8)
        for b in range(B):
            for m in range((int(lq[b]) + TILE - 1) // TILE):
                p_min = int(lkv[b] - lq[b]) + m * TILE
                p_max = int(lkv[b] - lq[b]) + min(m * TILE + TILE - 1, int(lq[b]) - 1)
                if p_max < 0:  # more queries than keys: this Q tile sees no key
                    continue
                lo = max(0, p_min // TILE - cfg.window)
                bm[b, :, m, lo:p_max // TILE + 1] = 1
    for (b, h, m) in cfg.zero_rows:
        bm[b, h, m, :] = 0
    del u
    # --- paging --------------------------------------------------------------
    pages_per_seq = (lkv + PS - 1) // PS
    NB = int(pages_per_seq.sum()) + spare_pages
    perm = np.arange(NB) if identity_pages else rng.permutation(NB)
    max_pages = int(pages_per_seq.max())
    spare = int(perm[-1]) if spare_pages > 0 else int(perm[0])
    block_table = np.full((B, max_pages), spare, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, :pages_per_seq[b]] = perm[off:off + pages_per_seq[b]]
        off += int(pages_per_seq[b])

    fill_code = NAN_CODE if fill == "nan" else 0
    fill_scale = np.float32(np.nan) if fill == "nan" else np.float32(0.0)
    if cfg.kv_layout == 0:
        shape, sshape = (NB, PS, Hkv, HEAD_DIM), (NB, PS, Hkv)
    else:
        shape, sshape = (NB, Hkv, PS, HEAD_DIM), (NB, Hkv, PS)
    kcache = np.full(shape, fill_code, dtype=np.uint8)
    vcache = np.full(shape, fill_code, dtype=np.uint8)
    kscale = np.full(sshape, fill_scale, dtype=np.float32) if cfg.quant_type == 1 else None
    start = 0
    for b in range(B):
        j = np.arange(int(lkv[b]))
        page = block_table[b, j // PS]
        slot = j % PS
        rows = slice(start, start + int(lkv[b]))
        if cfg.kv_layout == 0:
            kcache[page, slot] = kq[rows]
            vcache[page, slot] = vq[rows]
            if kscale is not None:
                kscale[page, slot] = ks_tok[rows]
        else:
            kcache[page, :, slot] = kq[rows]
            vcache[page, :, slot] = vq[rows]
            if kscale is not None:
                kscale[page, :, slot] = ks_tok[rows]
        start += int(lkv[b])
    if kscale is None:
        kscale = np.asarray(ks_tok[0, :1], dtype=np.float32).reshape(1).copy()

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lq)
    return Problem(cfg=cfg, q=q, kcache=kcache, vcache=vcache, qscale=qscale, kscale=kscale,
                   vscale=np.ascontiguousarray(vscale, dtype=np.float32), cu_seqlens_q=cu,
                   block_table=block_table, seqlens_kv=lkv.astype(np.int32),
                   block_mask=bm if mask else None, max_seqlen_q=int(lq.max()),
                   softmax_scale=1.0 / float(np.sqrt(HEAD_DIM)))


def sample_q_tiles(problem, count, seed=0, must_include=()):
    """`count` distinct (b, h, m) Q tiles chosen with a seeded RNG, plus `must_include`."""
    rng = np.random.default_rng(seed)
    lq = np.diff(problem.cu_seqlens_q)
    Hq = problem.q.shape[1]
    all_tiles = [(b, h, m) for b in range(len(lq)) for h in range(Hq)
                 for m in range(int((lq[b] + TILE - 1) // TILE))]
    pick = rng.choice(len(all_tiles), size=min(count, len(all_tiles)), replace=False)
    chosen = {all_tiles[i] for i in pick}
    chosen.update(tuple(t) for t in must_include)
    return sorted(chosen)


def index_form(problem, order="ascending", seed=0, junk=True):
    """The block mask of `problem` rewritten as per-Q-tile index lists (the index
    form of "Quant Block Sparse Attention", "Key parameters"): returns
    (sparse_indices int32 [B,Hq,Mt,Kb+2], sparse_seq_len int32 [B,Hq,Mt]).

    Every non-zero mask entry of a Q tile is listed once.  order: "ascending"
    or "shuffled" (seeded).  junk: also list two tiles that select nothing
    (-1 and a tile past the KV length) at seeded positions, and fill the
    unused tail of every list with arbitrary tile ids (which must be ignored).
    No arithmetic of the method happens here.
    """
    bm = problem.block_mask
    assert bm is not None
    B, Hq, Mt, Kb = bm.shape
    cap = Kb + 2
    rng = np.random.default_rng(seed)
    idx = rng.integers(-5, Kb + 5, size=(B, Hq, Mt, cap)).astype(np.int32)   # arbitrary tail
    seq_len = np.zeros((B, Hq, Mt), dtype=np.int32)
    for b in range(B):
        n_tiles = int((problem.seqlens_kv[b] + TILE - 1) // TILE)
        for h in range(Hq):
            for m in range(Mt):
                tiles = np.nonzero(bm[b, h, m])[0].astype(np.int32)
                if order == "shuffled":
                    tiles = rng.permutation(tiles)
                lst = list(tiles)
                if junk:
                    for bad in (-1, n_tiles + int(rng.integers(0, 3))):
                        lst.insert(int(rng.integers(0, len(lst) + 1)), bad)
                idx[b, h, m, :len(lst)] = lst
                seq_len[b, h, m] = len(lst)
    return idx, seq_len


def topk_index_form(problem, k, seed=0):
    """Index lists of a fixed capacity k that do not come from a mask: for every
    Q tile, min(k, ceil(Lkv/128)) distinct KV tiles drawn uniformly from the
    sequence's tiles, in seeded random order (a top-k style selection that
    ignores causality: tiles above the causal range select nothing).  Returns
    (sparse_indices int32 [B,Hq,Mt,k], sparse_seq_len int32 [B,Hq,Mt]), Mt as
    in the block mask."""
    B, Hq, Mt, _ = problem.block_mask.shape
    rng = np.random.default_rng(seed)
    idx = np.full((B, Hq, Mt, k), -1, dtype=np.int32)
    seq_len = np.zeros((B, Hq, Mt), dtype=np.int32)
    for b in range(B):
        n_tiles = int((problem.seqlens_kv[b] + TILE - 1) // TILE)
        take = min(k, n_tiles)
        for h in range(Hq):
            for m in range(Mt):
                idx[b, h, m, :take] = rng.permutation(n_tiles)[:take]
                seq_len[b, h, m] = take
    return idx, seq_len


def append_inputs(problem, seed=0, spread=True):
    """bfloat16 inputs of the quantise-and-append step for `problem`'s query
    chunk: the chunk's Q [T,Hq,128], and K and V [T,Hkv,128] for the same
    tokens (they land at the tail of each KV sequence), as float32 arrays
    holding bfloat16 values; plus static descales (kscale [1] for quant type
    0, vscale [1] or [Hkv]).  N(0,1) values times a per-row magnitude drawn
    log-uniformly from 2^-20 .. 2^20 (spread=True), with a few all-zero rows;
    the static descales are fixed numbers, so large rows saturate.  Only random
    draws and bfloat16 rounding (torch's CPU cast) happen here."""
    rng = np.random.default_rng(seed)
    T, Hq, _ = problem.q.shape
    Hkv = problem.cfg.hkv

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if spread:
            mag = np.exp2(rng.uniform(-20, 20, size=shape[:2])).astype(np.float32)
            x = x * mag[..., None]
            zero = rng.random(shape[:2]) < 0.01
            x[zero] = 0.0
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()

    q = draw((T, Hq, HEAD_DIM))
    k = draw((T, Hkv, HEAD_DIM))
    v = draw((T, Hkv, HEAD_DIM))
    kscale = np.array([0.0125], dtype=np.float32)
    if problem.quant_type == 1:
        vscale = rng.uniform(0.01, 0.015, size=Hkv).astype(np.float32)
    else:
        vscale = np.array([0.0117], dtype=np.float32)
    return dict(q=q, k=k, v=v, kscale=kscale, vscale=vscale)


def to_ntd(problem):
    """Q codes and Q descales in the NTD layout: [Hq,T,128] and [Hq,T]."""
    return (np.ascontiguousarray(problem.q.transpose(1, 0, 2)),
            np.ascontiguousarray(problem.qscale.T))
