"""fp64 CPU oracle of block-sparse FP8 attention prefill over a paged KV cache.

Test infrastructure only (see the package docstring).  Plain, slow NumPy in
float64; no blocking or reordering beyond what the definition states.

What is computed ("Quant Block Sparse Attention", section "Operator
introduction", the attention formula):

    Q^_i = Q_i^fp8 * q_descale_i
    K^_j = K_j^fp8 * k_descale_j
    V^_j = V_j^fp8 * v_descale_head(j)
    O_i  = sum_{j in Omega_i} softmax_{j in Omega_i}(Q^_i . K^_j * softmax_scale + mask_ij) V^_j

Readings adopted where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

  * Omega_i, the sparse KV set of query i, is every key position j with
    j < Lkv_b whose 128-token KV tile is switched on in the uint8 block mask of
    the query's 128-token Q tile (non-zero byte = compute, hpc-ops article,
    "Block-sparse scheduling"), intersected, in causal mode, with j <= p_i.
  * Causal alignment is bottom-right ("right-context causal", constraint
    table of "Quant Block Sparse Attention"): query t of a sequence with Lq
    queries and Lkv keys sits at position p = Lkv - Lq + t.
  * Q tiles count from the first query of each sequence; KV tiles from key 0.
  * GQA maps q-head h to kv-head h // (Hq / Hkv).
  * An empty Omega_i gives O_i = 0 and LSE_i = -FLT_MAX ("Sparse indices &
    PA page table": an empty sparse task outputs 0 with LSE -FLT_MAX).
  * LSE is the natural log of sum_j exp(score_j), laid out [Hq, T].
  * All scales are descales (multiplied in).
  * quant_type 0: K and V per-tensor (kscale[0], vscale[0]).
    quant_type 1: K per (token slot, kv-head), laid out like the cache minus
    the head dimension; V per kv-head.  (hpc-ops article, "FP8 Tensor Core
    compute": the two QuantType schemes; "Quant Block Sparse Attention", "Key
    parameters": k_descale per token/head, v_descale per kv-head.)

P-emulating mode ("emulate") follows the fixed P-scale of the hpc-ops article
("FP8 Tensor Core compute: fixed P-scale quantisation") together with the
active-tile loop of its "Active tile list" section: the active KV tiles of a Q
tile are visited in ascending order, 128 keys at a time, with an online softmax;
the probabilities of a tile, taken against the running maximum after that
tile, are multiplied by 256 and rounded to E4M3; the row sum uses the
unrounded probabilities; the final output divides by 256 once and applies the
V descale.  The output accumulation itself is done in float64.

Two input forms select the sparse KV tiles of a Q tile:
  * the uint8 block mask [B,Hq,Mt,Kb] (hpc-ops article), tiles visited in
    ascending order;
  * the index form of "Quant Block Sparse Attention" ("Key parameters",
    "Sparse indices & PA page table"): sparse_indices [B,Hq,Mt,Kb] int32 lists
    logical KV tiles, of which the first sparse_seq_len[b,h,m] are valid.  The
    set of listed tiles is the sparse set; the emulating mode visits them in
    list order.  Entries outside [0, ceil(Lkv/128)) select nothing.
The probability scale of the emulating mode is p_scale ("Key parameters":
p_scale, a positive finite probability quantisation scale), 256 when not
given.  Q may come in the TND layout [T,Hq,128] with q_descale [T,Hq] or in the
NTD layout [Hq,T,128] with q_descale [Hq,T] ("Key parameters": query and
q_descale layouts); the output is TND either way.
"""
import numpy as np

from . import e4m3

TILE = 128
HEAD_DIM = 128
NEG_FLT_MAX = -3.4028234663852886e38   # -FLT_MAX, the LSE of an empty sparse set

NHD = 0   # kcache/vcache [num_pages, page_size, Hkv, 128]
HND = 1   # kcache/vcache [num_pages, Hkv, page_size, 128]

TND = 0   # q [T, Hq, 128], qscale [T, Hq]
NTD = 1   # q [Hq, T, 128], qscale [Hq, T]

DEFAULT_P_SCALE = 256.0


def _ceil_div(a, b):
    return (a + b - 1) // b


def _dequant_kv_sequence(cache, scale, block_table_row, lkv, g, page_size, kv_layout,
                         per_token_scale, vector_scale):
    """Dequantised K^ (or V^) rows 0..lkv-1 of one sequence and kv-head g.

    Logical key j lives in logical page j // page_size at slot j % page_size;
    the page table maps the logical page to a physical page ("Quant Block
    Sparse Attention", "Sparse indices & PA page table"; hpc-ops article,
    "Quick start": the KV cache is paged and block_ids is the page table).
    Only pages that hold keys below lkv are read.
    """
    j = np.arange(lkv)
    page = block_table_row[j // page_size]
    slot = j % page_size
    if kv_layout == NHD:
        codes = cache[page, slot, g, :]
    else:
        codes = cache[page, g, slot, :]
    vals = e4m3.decode(codes)
    if per_token_scale:
        s = scale[page, slot, g] if kv_layout == NHD else scale[page, g, slot]
        vals = vals * np.asarray(s, dtype=np.float64)[:, None]
    else:
        vals = vals * np.float64(vector_scale)
    return vals


def _sequence_bounds(cu_seqlens_q, seqlens_kv, b):
    t0 = int(cu_seqlens_q[b])
    lq = int(cu_seqlens_q[b + 1]) - t0
    lkv = int(seqlens_kv[b])
    return t0, lq, lkv


def _listed_tiles(sparse_indices, sparse_seq_len, b, h, m, n_tiles):
    """Valid entries of the index list of Q tile m, in list order."""
    length = int(sparse_seq_len[b, h, m])
    entries = np.asarray(sparse_indices[b, h, m, :max(length, 0)], dtype=np.int64)
    return entries[(entries >= 0) & (entries < n_tiles)]


def _tile_keys(block_mask, b, h, m, lkv, index_form=None):
    """KV tiles selected for Q tile m (in visiting order) and their key
    positions (< lkv), tile by tile."""
    n_tiles = _ceil_div(lkv, TILE)
    if index_form is not None:
        tiles = _listed_tiles(index_form[0], index_form[1], b, h, m, n_tiles)
    elif block_mask is None:
        tiles = np.arange(n_tiles)             # no mask: the dense path, every tile
    else:
        row = np.asarray(block_mask[b, h, m, :n_tiles])
        on = np.zeros(n_tiles, dtype=bool)
        on[: row.shape[0]] = row != 0
        tiles = np.nonzero(on)[0]
    if tiles.size == 0:
        return tiles, np.zeros(0, dtype=np.int64)
    keys = (tiles[:, None] * TILE + np.arange(TILE)[None, :]).reshape(-1)
    return tiles, keys[keys < lkv]


def _q_tile(inp, b, h, m, mode, kcache_deq, vcache_deq):
    """Outputs of one (sequence b, q-head h, Q tile m): O [rows,128], LSE [rows]."""
    t0, lq, lkv = _sequence_bounds(inp["cu_seqlens_q"], inp["seqlens_kv"], b)
    rows = np.arange(TILE * m, min(TILE * m + TILE, lq))
    q = e4m3.decode(inp["q"][t0 + rows, h, :]) * \
        np.asarray(inp["qscale"][t0 + rows, h], dtype=np.float64)[:, None]
    tiles, keys = _tile_keys(inp["block_mask"], b, h, m, lkv, inp["index_form"])
    khat = kcache_deq[keys]
    vhat = vcache_deq[keys]
    scores = inp["softmax_scale"] * (q @ khat.T)                     # [rows, keys]
    allowed = np.ones(scores.shape, dtype=bool)
    if inp["causal"]:
        p = lkv - lq + rows                                           # bottom-right alignment
        allowed = keys[None, :] <= p[:, None]
    scores = np.where(allowed, scores, -np.inf)

    o = np.zeros((rows.size, HEAD_DIM))
    lse = np.full(rows.size, NEG_FLT_MAX)
    nonempty = allowed.any(axis=1)
    if mode == "exact":
        mx = np.where(nonempty, scores.max(axis=1, initial=-np.inf), 0.0)
        w = np.exp(scores - mx[:, None])                              # exp(-inf) = 0
        lsum = w.sum(axis=1)
        o[nonempty] = (w @ vhat)[nonempty] / lsum[nonempty, None]
        lse[nonempty] = mx[nonempty] + np.log(lsum[nonempty])
        return rows, o, lse

    # P-emulating mode: active tiles in visiting order, 128 keys each, online softmax.
    vcodes = inp["_vcodes_cache"][keys]                               # V^fp8 values (no descale)
    run_max = np.full(rows.size, -np.inf)
    run_sum = np.zeros(rows.size)
    acc = np.zeros((rows.size, HEAD_DIM))
    key_tile = keys // TILE
    for n in tiles:
        cols = np.nonzero(key_tile == n)[0]
        if cols.size == 0:
            continue
        s = scores[:, cols]
        new_max = np.maximum(run_max, s.max(axis=1))
        safe_new = np.where(np.isfinite(new_max), new_max, 0.0)        # all keys so far masked
        alpha = np.where(np.isfinite(run_max), np.exp(run_max - safe_new), 0.0)
        p_tilde = np.exp(s - safe_new[:, None])                        # masked -> 0
        p8 = e4m3.round_to_grid(inp["p_scale"] * p_tilde)              # P-scale, then E4M3
        run_sum = alpha * run_sum + p_tilde.sum(axis=1)
        acc = alpha[:, None] * acc + p8 @ vcodes[cols]
        run_max = new_max
    vs = inp["_vscale_g"]
    o[nonempty] = acc[nonempty] * vs / (inp["p_scale"] * run_sum[nonempty, None])
    lse[nonempty] = run_max[nonempty] + np.log(run_sum[nonempty])
    return rows, o, lse


def prefill(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
            seqlens_kv, block_mask, quant_type, page_size, kv_layout=NHD,
            softmax_scale=None, causal=True, mode="exact", tiles=None,
            sparse_indices=None, sparse_seq_len=None, p_scale=None, q_layout=TND):
    """Oracle of the whole prefill.

    Arrays are NumPy: q uint8 [T,Hq,128] (E4M3 codes); kcache/vcache uint8
    codes in NHD or HND paged layout; qscale float32 [T,Hq]; kscale float32
    [1] (quant 0) or per slot (quant 1); vscale float32 [1] (quant 0) or
    [Hkv] (quant 1); cu_seqlens_q int32 [B+1]; block_table int32 [B,pages];
    seqlens_kv int32 [B]; block_mask uint8 [B,Hq,Mt,Kb] or None.

    mode: "exact" (the formula in float64) or "emulate" (P-scale, 256 unless
    p_scale is given, with E4M3 rounding of P, see the module docstring).
    tiles: optional iterable of (b, h, m) Q tiles to compute; every other
    output element is left NaN.  Default: every Q tile of every sequence.
    sparse_indices / sparse_seq_len: the index form (block_mask must be None).
    q_layout: TND or NTD for q and qscale.

    Returns (O float64 [T,Hq,128], LSE float64 [Hq,T]).
    """
    q = np.asarray(q)
    qscale = np.asarray(qscale)
    if q_layout == NTD:                      # [Hq,T,128] and [Hq,T]: same values, axes swapped
        q = q.transpose(1, 0, 2)
        qscale = qscale.T
    index_form = None
    if sparse_indices is not None:
        assert block_mask is None, "give either the block mask or the index form"
        index_form = (np.asarray(sparse_indices), np.asarray(sparse_seq_len))
    T, Hq, D = q.shape
    assert D == HEAD_DIM
    Hkv = kcache.shape[2] if kv_layout == NHD else kcache.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(HEAD_DIM)
    B = len(seqlens_kv)
    inp = dict(q=q, qscale=qscale, cu_seqlens_q=np.asarray(cu_seqlens_q),
               seqlens_kv=np.asarray(seqlens_kv), block_mask=block_mask,
               softmax_scale=float(softmax_scale), causal=bool(causal), index_form=index_form,
               p_scale=float(DEFAULT_P_SCALE if p_scale is None else p_scale))
    out = np.full((T, Hq, HEAD_DIM), np.nan)
    lse = np.full((Hq, T), np.nan)

    if tiles is None:
        tiles = []
        for b in range(B):
            _, lq, _ = _sequence_bounds(inp["cu_seqlens_q"], inp["seqlens_kv"], b)
            for h in range(Hq):
                for m in range(_ceil_div(lq, TILE)):
                    tiles.append((b, h, m))
    by_bg = {}
    for (b, h, m) in tiles:
        by_bg.setdefault((b, h // group), []).append((h, m))

    per_token = quant_type == 1
    for (b, g), work in sorted(by_bg.items()):
        t0, lq, lkv = _sequence_bounds(inp["cu_seqlens_q"], inp["seqlens_kv"], b)
        bt = np.asarray(block_table[b])
        k_deq = _dequant_kv_sequence(kcache, kscale, bt, lkv, g, page_size, kv_layout,
                                     per_token, None if per_token else kscale[0])
        v_scale_g = float(vscale[g] if per_token else vscale[0])
        v_codes = _dequant_kv_sequence(vcache, None, bt, lkv, g, page_size, kv_layout,
                                       False, 1.0)
        v_deq = v_codes * v_scale_g
        inp["_vcodes_cache"] = v_codes
        inp["_vscale_g"] = v_scale_g
        for (h, m) in work:
            rows, o, l = _q_tile(inp, b, h, m, mode, k_deq, v_deq)
            out[t0 + rows, h, :] = o
            lse[h, t0 + rows] = l
    return out, lse


def brute_force(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
                seqlens_kv, block_mask, quant_type, page_size, kv_layout=NHD,
                softmax_scale=None, causal=True, sparse_indices=None, sparse_seq_len=None,
                q_layout=TND):
    """Full-matrix reference for tiny shapes: every (query, key) pair is scored
    and masked element by element, then a plain softmax is taken per row.

    The KV sequence is first unpacked from the paged cache into a dense
    [Lkv, Hkv, 128] array by walking the page table slot by slot, and the mask
    decision for pair (t, j) is made from the definition of Omega alone:
    block_mask[b, h, t // 128, j // 128] != 0 (index form: j // 128 is one of
    the first sparse_seq_len[b, h, t // 128] entries of the list), j < Lkv, and
    (causal) j <= p_t.  In the NTD layout q[h, t] and qscale[h, t] are read.
    """
    q = np.asarray(q)
    if q_layout == NTD:
        def q_at(t, h):
            return q[h, t], qscale[h, t]
        T = q.shape[1]
    else:
        def q_at(t, h):
            return q[t, h], qscale[t, h]
        T = q.shape[0]
    Hq, D = (q.shape[0], q.shape[2]) if q_layout == NTD else (q.shape[1], q.shape[2])
    Hkv = kcache.shape[2] if kv_layout == NHD else kcache.shape[1]
    group = Hq // Hkv
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(D)
    out = np.zeros((T, Hq, D))
    lse = np.zeros((Hq, T))
    for b in range(len(seqlens_kv)):
        t0 = int(cu_seqlens_q[b])
        lq = int(cu_seqlens_q[b + 1]) - t0
        lkv = int(seqlens_kv[b])
        kd = np.zeros((lkv, Hkv, D))
        vd = np.zeros((lkv, Hkv, D))
        for j in range(lkv):
            page = int(block_table[b][j // page_size])
            slot = j % page_size
            for g in range(Hkv):
                if kv_layout == NHD:
                    kc, vc = kcache[page, slot, g], vcache[page, slot, g]
                else:
                    kc, vc = kcache[page, g, slot], vcache[page, g, slot]
                if quant_type == 1:
                    ks = kscale[page, slot, g] if kv_layout == NHD else kscale[page, g, slot]
                    vs = vscale[g]
                else:
                    ks, vs = kscale[0], vscale[0]
                kd[j, g] = e4m3.decode(kc) * float(ks)
                vd[j, g] = e4m3.decode(vc) * float(vs)
        for h in range(Hq):
            g = h // group
            for t in range(lq):
                qc, qs = q_at(t0 + t, h)
                qv = e4m3.decode(qc) * float(qs)
                p = lkv - lq + t
                allowed = np.zeros(lkv, dtype=bool)
                for j in range(lkv):
                    if sparse_indices is not None:
                        n_valid = int(sparse_seq_len[b, h, t // TILE])
                        on = any(int(sparse_indices[b, h, t // TILE, k]) == j // TILE for k in range(n_valid))
                    else:
                        on = True if block_mask is None else block_mask[b, h, t // TILE, j // TILE] != 0
                    allowed[j] = on and ((not causal) or j <= p)
                if not allowed.any():
                    out[t0 + t, h] = 0.0
                    lse[h, t0 + t] = NEG_FLT_MAX
                    continue
                s = softmax_scale * (kd[allowed, g] @ qv)
                mx = s.max()
                w = np.exp(s - mx)
                out[t0 + t, h] = (w[:, None] * vd[allowed, g]).sum(axis=0) / w.sum()
                lse[h, t0 + t] = mx + np.log(w.sum())
    return out, lse


def round_bf16(x):
    """Round float64 to the nearest bfloat16 value (RNE), returned as float64.

    bfloat16 keeps 8 significant bits and fp32's exponent range; the output
    data type is BF16 ("Quant Block Sparse Attention", constraint table).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, E = np.frexp(a)
    e = np.maximum(E - 1, -126)
    qstep = np.ldexp(1.0, e - 7)
    r = np.rint(a / qstep) * qstep
    r = np.where(np.isfinite(x), r, x)
    return np.copysign(r, x)
