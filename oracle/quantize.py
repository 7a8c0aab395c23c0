"""Oracle of the FP8 quantise-and-append step that produces the prefill's inputs.

Test infrastructure only (see the package docstring).  Plain NumPy.

What is computed (the method of the FlashMLA FP8 KV-cache article, section
"Quant/dequant source": every 1x128 tile of a row gets the scale
max|x| / 448, optionally rounded up to a power of two, and the stored value is
the E4M3 value of x divided by that scale; the scale is the descale the kernel
multiplies back in):

  * a row is the 128 head-dim values of one (token, head);
  * descale d = fp32(amax / 448) with amax = max |x| over the row, the
    division in float32 (the precision of the reference, whose inputs are
    bfloat16 and whose arithmetic is float32); with pow2, d is rounded up to
    the next power of two (a power of two stays);
  * code = E4M3(fp32(x / d)), round to nearest even, saturating at 448;
  * a row of zeros has amax = 0: d = 1 and every code is 0 (any descale
    reproduces zeros; 1 keeps later arithmetic finite).

Which rows get a computed descale follows the prefill's quantisation schemes
(hpc-ops article, "FP8 Tensor Core compute", the two QuantType values; "Quant
Block Sparse Attention", "Key parameters"): Q per (token, head) always; K per
(token, kv-head) for quant type 1, else K with the given per-tensor descale;
V with the given descale (per tensor for quant type 0, per kv-head for 1).  A
given descale is used as d in the same code formula.

Appending ("Quant Block Sparse Attention", "Key parameters" and "Sparse indices
& PA page table": paged cache through the block table; the query chunk sits at
the tail of the KV sequence, right-context causal): the new tokens of sequence
b are its Lq_b queries, and token i of the chunk is stored at logical position
p = Lkv_b - Lq_b + i, i.e. physical page block_table[b, p // page_size], slot
p % page_size, in the NHD or HND layout.  Per-token K descales (quant type 1)
go to the same (page, slot, kv-head) place of the descale array.
"""
import numpy as np

from . import e4m3

HEAD_DIM = 128
FP8_MAX = 448.0
NHD = 0
HND = 1


def row_descale(x, pow2=False):
    """float32 descales of rows x [..., 128] (float32 values)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    d = amax / np.float32(FP8_MAX)                    # float32 division
    d = np.where(amax == 0, np.float32(1.0), d).astype(np.float32)
    if pow2:
        m, e = np.frexp(d.astype(np.float64))          # d = m * 2^e, m in [0.5, 1)
        d = np.where(m == 0.5, d, np.ldexp(1.0, e)).astype(np.float32)
    return d


def encode_with(x, d):
    """E4M3 codes of fp32(x / d); d broadcasts over the last axis."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(d, dtype=np.float32)[..., None]
    return e4m3.encode(q.astype(np.float64))


def quantize_rows(x, pow2=False):
    """(codes uint8 [..., 128], descale float32 [...]) of rows with computed descales."""
    d = row_descale(x, pow2)
    return encode_with(x, d), d


def quantize_append(q, k, v, cu_seqlens_q, seqlens_kv, block_table, kscale, vscale,
                    quant_type, page_size, kv_layout, kcache, vcache, kscale_cache=None,
                    pow2=False):
    """Quantise Q and append the chunk's K and V to copies of the caches.

    q [T,Hq,128], k and v [T,Hkv,128]: float32 arrays holding bfloat16 values.
    kscale: float32 [1], the K descale of quant type 0 (unused for type 1).
    vscale: float32 [1] (type 0) or [Hkv] (type 1).
    kcache / vcache: uint8 paged caches; kscale_cache: float32 cache-shaped
    descales without the head dimension (type 1).
    Returns (q_codes [T,Hq,128], qscale [T,Hq], kcache, vcache, kscale_cache).
    """
    q_codes, qscale = quantize_rows(q, pow2)
    kcache = np.array(kcache, copy=True)
    vcache = np.array(vcache, copy=True)
    kscale_cache = None if kscale_cache is None else np.array(kscale_cache, copy=True)
    if quant_type == 1:
        k_codes, k_d = quantize_rows(k, pow2)
        v_d = np.broadcast_to(np.asarray(vscale, dtype=np.float32)[None, :], k.shape[:2])
    else:
        k_d = np.full(k.shape[:2], np.float32(np.asarray(kscale).reshape(-1)[0]))
        k_codes = encode_with(k, k_d)
        v_d = np.full(k.shape[:2], np.float32(np.asarray(vscale).reshape(-1)[0]))
    v_codes = encode_with(v, v_d)

    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lkv = np.asarray(seqlens_kv, dtype=np.int64)
    for b in range(len(lkv)):
        lq = int(cu[b + 1] - cu[b])
        for i in range(lq):
            t = int(cu[b]) + i
            pos = int(lkv[b]) - lq + i
            page = int(block_table[b, pos // page_size])
            slot = pos % page_size
            if kv_layout == NHD:
                kcache[page, slot] = k_codes[t]
                vcache[page, slot] = v_codes[t]
                if quant_type == 1:
                    kscale_cache[page, slot] = k_d[t]
            else:
                kcache[page, :, slot] = k_codes[t]
                vcache[page, :, slot] = v_codes[t]
                if quant_type == 1:
                    kscale_cache[page, :, slot] = k_d[t]
    return q_codes, qscale, kcache, vcache, kscale_cache
