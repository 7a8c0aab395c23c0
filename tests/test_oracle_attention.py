"""Pins of the fp64 attention oracle against brute force, a library special case,
closed forms and invariances.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import e4m3
from synth import make_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CONSTRAINTS = json.load(open(os.path.join(GOLDEN, "constraints.json")))
NEG_FLT_MAX = CONSTRAINTS["empty_set"]["lse"]

# Small shapes spanning several tiles, ragged tails, varlen chunked prefill,
# GQA, both quant types, both layouts and both page sizes.
SMALL = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(129,), lkv=(383,), hq=3, hkv=3, quant_type=1, kv_layout=0, page_size=32, keep=0.3),
    dict(lq=(64, 256), lkv=(250, 256), hq=4, hkv=1, quant_type=0, kv_layout=1, page_size=64, keep=0.7),
]


def small_problem(i, seed=7, **kw):
    return make_problem("tiny", seed=seed + i, **{**SMALL[i], **kw})


def omega_sizes(p):
    """|Omega_t| per (h, token), counted element by element from the definition."""
    T, Hq, _ = p.q.shape
    out = np.zeros((Hq, T), dtype=np.int64)
    for b in range(len(p.seqlens_kv)):
        t0, t1 = p.cu_seqlens_q[b], p.cu_seqlens_q[b + 1]
        lq, lkv = t1 - t0, p.seqlens_kv[b]
        for h in range(Hq):
            for t in range(lq):
                cnt = 0
                for j in range(lkv):
                    on = p.block_mask is None or p.block_mask[b, h, t // 128, j // 128] != 0
                    if on and (not p.causal or j <= lkv - lq + t):
                        cnt += 1
                out[h, t0 + t] = cnt
    return out


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_exact_matches_brute_force(i):
    p = small_problem(i, fill="nan")
    o, l = A.prefill(**p.oracle_kwargs(), mode="exact")
    ob, lb = A.brute_force(**p.oracle_kwargs())
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_exact_matches_brute_force_non_causal():
    p = small_problem(1)
    kw = {**p.oracle_kwargs(), "causal": False}
    o, l = A.prefill(**kw, mode="exact")
    ob, lb = A.brute_force(**kw)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def dequant_dense(p, b):
    """Dense [Lkv, Hkv, 128] K^ and V^ of sequence b via torch (independent of the oracle codec)."""
    lkv, PS = int(p.seqlens_kv[b]), p.page_size
    j = np.arange(lkv)
    page, slot = p.block_table[b, j // PS], j % PS
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double()  # noqa
    if p.kv_layout == 0:
        kc, vc = p.kcache[page, slot], p.vcache[page, slot]
        ks = p.kscale[page, slot] if p.quant_type == 1 else None
    else:
        kc, vc = p.kcache[page, :, slot], p.vcache[page, :, slot]
        ks = p.kscale[page, :, slot] if p.quant_type == 1 else None
    k = dec(kc) * (torch.from_numpy(ks).double()[..., None] if ks is not None else float(p.kscale[0]))
    vs = torch.from_numpy(p.vscale).double()
    v = dec(vc) * (vs[None, :, None] if p.quant_type == 1 else float(p.vscale[0]))
    return k, v


@pytest.mark.parametrize("i", [0, 1, 3])
def test_all_true_mask_equals_sdpa(i):
    """With every mask byte on, the method is dense causal attention: compare with
    torch's scaled_dot_product_attention (fp64, explicit bottom-right mask)."""
    p = small_problem(i)
    p.block_mask[:] = 1
    o, l = A.prefill(**p.oracle_kwargs(), mode="exact")
    Hq = p.q.shape[1]
    group = Hq // (p.kcache.shape[2] if p.kv_layout == 0 else p.kcache.shape[1])
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lq, lkv = t1 - t0, int(p.seqlens_kv[b])
        k, v = dequant_dense(p, b)
        q = torch.from_numpy(p.q[t0:t1].copy()).view(torch.float8_e4m3fn).double() * \
            torch.from_numpy(p.qscale[t0:t1]).double()[..., None]
        k = k.repeat_interleave(group, dim=1)
        v = v.repeat_interleave(group, dim=1)
        allowed = torch.arange(lkv)[None, :] <= (lkv - lq + torch.arange(lq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), attn_mask=allowed,
            scale=p.softmax_scale)
        np.testing.assert_allclose(o[t0:t1], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
        scores = torch.einsum("hqd,hkd->hqk", q.transpose(0, 1), k.transpose(0, 1)) * p.softmax_scale
        lse_ref = torch.logsumexp(scores.masked_fill(~allowed, -np.inf), dim=-1)
        np.testing.assert_allclose(l[:, t0:t1], lse_ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["exact", "emulate"])
def test_empty_sets(mode):
    p = small_problem(1)
    # (a) an all-zero mask row: every query of that Q tile has an empty set
    p.block_mask[1, 2, 0, :] = 0
    # (b) a row that keeps only a tile in the future of some of its queries:
    # sequence 0 has Lq=200, Lkv=390 -> Q tile 0 sits at positions 190..317,
    # so keeping only KV tile 2 (keys 256..383) leaves queries with p < 256 empty.
    p.block_mask[0, 1, 0, :] = 0
    p.block_mask[0, 1, 0, 2] = 1
    o, l = A.prefill(**p.oracle_kwargs(), mode=mode)
    t0b1 = int(p.cu_seqlens_q[1])
    assert np.all(o[t0b1:t0b1 + 77, 2] == 0.0)
    assert np.all(l[2, t0b1:t0b1 + 77] == NEG_FLT_MAX)
    lq, lkv = 200, 390
    pos = lkv - lq + np.arange(128)
    empty = pos < 256
    assert empty.any() and (~empty).any()
    assert np.all(o[:128][empty, 1] == 0.0)
    assert np.all(l[1, :128][empty] == NEG_FLT_MAX)
    assert np.all(l[1, :128][~empty] > NEG_FLT_MAX)
    # a mask holding only future tiles for the whole Q tile: output 0, LSE -FLT_MAX
    sizes = omega_sizes(p)
    assert np.all((l == NEG_FLT_MAX) == (sizes == 0))


@pytest.mark.parametrize("mode", ["exact", "emulate"])
def test_nan_in_unreferenced_pages_has_no_effect(mode):
    """Pages that no active tile touches, unused slots and spare pages can hold NaN."""
    cfg = dict(lq=(128,), lkv=(512,), hq=2, hkv=1, quant_type=1, kv_layout=0, page_size=64, keep=1.0)
    base = make_problem("tiny", seed=3, identity_pages=True, fill="zero", **cfg)
    nanp = make_problem("tiny", seed=3, identity_pages=True, fill="nan", **cfg)
    for p in (base, nanp):
        p.block_mask[:, :, :, 1] = 0       # KV tile 1 (keys 128..255) switched off everywhere
    # pages 2 and 3 (64-key pages) hold keys 128..255: poison them in the NaN copy
    nanp.kcache[2:4] = 0x7F
    nanp.vcache[2:4] = 0x7F
    nanp.kscale[2:4] = np.nan
    o0, l0 = A.prefill(**base.oracle_kwargs(), mode=mode)
    o1, l1 = A.prefill(**nanp.oracle_kwargs(), mode=mode)
    assert np.all(np.isfinite(o1))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


@pytest.mark.parametrize("mode", ["exact", "emulate"])
@pytest.mark.parametrize("i", [0, 1, 2])
def test_zero_q_closed_form(mode, i):
    """Q = 0 makes every score 0: LSE_t = ln|Omega_t| and O_t = mean of V^ over Omega_t.
    In emulate mode P' = 256 * 1 is exact in E4M3, so the same holds."""
    p = small_problem(i)
    p.q[:] = 0
    o, l = A.prefill(**p.oracle_kwargs(), mode=mode)
    sizes = omega_sizes(p)
    nz = sizes > 0
    np.testing.assert_allclose(l[nz], np.log(sizes[nz]), rtol=0, atol=1e-12)
    assert np.all(l[~nz] == NEG_FLT_MAX)
    # mean of V^ over Omega_t via cumulative sums of the dense dequantised V
    Hq = p.q.shape[1]
    Hkv = p.kcache.shape[2] if p.kv_layout == 0 else p.kcache.shape[1]
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lq, lkv = t1 - t0, int(p.seqlens_kv[b])
        _, v = dequant_dense(p, b)
        v = v.numpy()
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for t in range(0, lq, 37):
                keys = [j for j in range(lkv)
                        if p.block_mask[b, h, t // 128, j // 128] and j <= lkv - lq + t]
                want = v[keys, g].mean(axis=0) if keys else np.zeros(128)
                np.testing.assert_allclose(o[t0 + t, h], want, rtol=0, atol=1e-12)


def test_constant_v_closed_form():
    p = small_problem(0)
    p.vcache[:] = 0x38                      # every V code is 1.0
    o, _ = A.prefill(**p.oracle_kwargs(), mode="exact")
    np.testing.assert_allclose(o, float(p.vscale[0]), rtol=1e-13, atol=0)


def test_page_permutation_invariance():
    a = make_problem("tiny", seed=5, identity_pages=True, **SMALL[1])
    b = make_problem("tiny", seed=5, identity_pages=False, **SMALL[1])
    assert not np.array_equal(a.block_table, b.block_table)
    for mode in ("exact", "emulate"):
        oa, la = A.prefill(**a.oracle_kwargs(), mode=mode)
        ob, lb = A.prefill(**b.oracle_kwargs(), mode=mode)
        np.testing.assert_array_equal(oa, ob)
        np.testing.assert_array_equal(la, lb)


def test_gqa_equals_replicated_mha():
    p = small_problem(3)                    # Hq=4, Hkv=1, HND
    assert p.kv_layout == 1
    group = 4
    m = make_problem("tiny", seed=10, **SMALL[3])
    m.kcache = np.repeat(p.kcache, group, axis=1)
    m.vcache = np.repeat(p.vcache, group, axis=1)
    m.kscale, m.vscale = p.kscale, p.vscale
    m.q, m.qscale, m.block_mask, m.block_table = p.q, p.qscale, p.block_mask, p.block_table
    for mode in ("exact", "emulate"):
        o1, l1 = A.prefill(**p.oracle_kwargs(), mode=mode)
        o2, l2 = A.prefill(**m.oracle_kwargs(), mode=mode)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_quant1_with_uniform_scales_equals_quant0():
    p1 = small_problem(0, quant_type=1)
    p0 = small_problem(0, quant_type=0)
    p1.q, p1.qscale = p0.q, p0.qscale
    p1.kcache, p1.vcache = p0.kcache, p0.vcache
    p1.kscale = np.full_like(p1.kscale, p0.kscale[0])
    p1.vscale = np.full_like(p1.vscale, p0.vscale[0])
    p1.block_mask, p1.block_table = p0.block_mask, p0.block_table
    for mode in ("exact", "emulate"):
        o0, l0 = A.prefill(**p0.oracle_kwargs(), mode=mode)
        o1, l1 = A.prefill(**p1.oracle_kwargs(), mode=mode)
        np.testing.assert_allclose(o0, o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l0, l1, rtol=0, atol=1e-14)


def test_sequence_alone_equals_batched():
    p = small_problem(1)
    o, l = A.prefill(**p.oracle_kwargs(), mode="emulate")
    for b in range(2):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        kw = p.oracle_kwargs()
        kw.update(q=p.q[t0:t1], qscale=p.qscale[t0:t1], cu_seqlens_q=np.array([0, t1 - t0], np.int32),
                  block_table=p.block_table[b:b + 1], seqlens_kv=p.seqlens_kv[b:b + 1],
                  block_mask=p.block_mask[b:b + 1])
        ob, lb = A.prefill(**kw, mode="emulate")
        np.testing.assert_array_equal(o[t0:t1], ob)
        np.testing.assert_array_equal(l[:, t0:t1], lb)


def test_null_mask_equals_all_ones():
    p = small_problem(2)
    kw = p.oracle_kwargs()
    ones = np.ones_like(p.block_mask)
    for mode in ("exact", "emulate"):
        o1, l1 = A.prefill(**{**kw, "block_mask": None}, mode=mode)
        o2, l2 = A.prefill(**{**kw, "block_mask": ones}, mode=mode)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def emulate_scalar(p, b, h, t):
    """P-emulating reference for one query in scalar Python: tiles ascending,
    running max, P rounded by torch's float8_e4m3fn cast of 256*P (a library
    rounding independent of the oracle's codec; values are <= 256 so the cast
    cannot saturate), fp64 accumulation."""
    t0 = int(p.cu_seqlens_q[b])
    lq = int(p.cu_seqlens_q[b + 1]) - t0
    lkv = int(p.seqlens_kv[b])
    Hq = p.q.shape[1]
    Hkv = p.kcache.shape[2] if p.kv_layout == 0 else p.kcache.shape[1]
    g = h // (Hq // Hkv)
    k, _ = dequant_dense(p, b)
    k = k.numpy()
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()  # noqa
    q = dec(p.q[t0 + t, h]) * float(p.qscale[t0 + t, h])
    j = np.arange(lkv)
    page, slot = p.block_table[b, j // p.page_size], j % p.page_size
    vcodes = dec(p.vcache[page, slot, g] if p.kv_layout == 0 else p.vcache[page, g, slot])
    vs = float(p.vscale[g] if p.quant_type == 1 else p.vscale[0])
    run_max, run_sum, acc = -np.inf, 0.0, np.zeros(128)
    for n in range((lkv + 127) // 128):
        if p.block_mask[b, h, t // 128, n] == 0:
            continue
        keys = [jj for jj in range(n * 128, min(n * 128 + 128, lkv)) if jj <= lkv - lq + t]
        if not keys:
            continue
        s = [p.softmax_scale * float(np.dot(q, k[jj, g])) for jj in keys]
        new_max = max(run_max, max(s))
        alpha = np.exp(run_max - new_max) if np.isfinite(run_max) else 0.0
        pt = [np.exp(x - new_max) for x in s]
        p8 = torch.tensor([256.0 * x for x in pt], dtype=torch.float64).to(torch.float8_e4m3fn).double().numpy()
        run_sum = alpha * run_sum + sum(pt)
        acc = alpha * acc
        for w8, jj in zip(p8, keys):
            acc = acc + w8 * vcodes[jj]
        run_max = new_max
    if run_sum == 0:
        return np.zeros(128), NEG_FLT_MAX
    return acc * vs / (256.0 * run_sum), run_max + np.log(run_sum)


@pytest.mark.parametrize("i", [1, 2])
def test_emulate_matches_scalar_reference(i):
    p = small_problem(i)
    o, l = A.prefill(**p.oracle_kwargs(), mode="emulate")
    rng = np.random.default_rng(i)
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        for t in rng.choice(t1 - t0, size=min(6, t1 - t0), replace=False):
            for h in range(p.q.shape[1]):
                ow, lw = emulate_scalar(p, b, h, int(t))
                np.testing.assert_allclose(o[t0 + t, h], ow, rtol=0, atol=1e-12)
                np.testing.assert_allclose(l[h, t0 + t], lw, rtol=0, atol=1e-12)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_emulate_error_bound(i):
    """Rounding 256*P to E4M3 moves each weight by at most half an E4M3 spacing:
    <= 2^-4 relative in the normal range and <= 2^-10 absolute (in units of
    256*P) below it.  Hence |O_emul - O_exact| <= sum_j max(2^-4 P_j, 2^-18) |V^_j| / l,
    with P_j = exp(s_j - max) and l = sum_j P_j; LSE is unchanged by the rounding."""
    p = small_problem(i)
    oe, le = A.prefill(**p.oracle_kwargs(), mode="exact")
    om, lm = A.prefill(**p.oracle_kwargs(), mode="emulate")
    np.testing.assert_allclose(lm, le, rtol=0, atol=1e-12)
    Hq = p.q.shape[1]
    Hkv = p.kcache.shape[2] if p.kv_layout == 0 else p.kcache.shape[1]
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lq, lkv = t1 - t0, int(p.seqlens_kv[b])
        k, v = dequant_dense(p, b)
        k, v = k.numpy(), v.numpy()
        for h in range(Hq):
            g = h // (Hq // Hkv)
            q = e4m3.decode(p.q[t0:t1, h]) * p.qscale[t0:t1, h, None].astype(np.float64)
            s = p.softmax_scale * q @ k[:, g].T
            tiles_on = p.block_mask[b, h][np.arange(lq) // 128][:, np.arange(lkv) // 128] != 0
            allowed = tiles_on & (np.arange(lkv)[None, :] <= (lkv - lq + np.arange(lq))[:, None])
            s = np.where(allowed, s, -np.inf)
            mx = np.where(allowed.any(1), s.max(1), 0.0)
            pw = np.exp(s - mx[:, None])
            l = pw.sum(1)
            ok = l > 0
            bound = (np.maximum(2.0 ** -4 * pw, 2.0 ** -18 * allowed) @ np.abs(v[:, g]))[ok] / l[ok, None]
            diff = np.abs(om[t0:t1, h] - oe[t0:t1, h])[ok]
            assert np.all(diff <= bound + 1e-12)
    rel = np.sqrt(np.mean((om - oe) ** 2) / np.mean(oe ** 2))
    assert 1e-3 < rel < 5e-2      # the rounding happened, and is of E4M3's size
    assert np.abs(om - oe).max() <= 0.1


def test_tiles_argument_computes_only_those_tiles():
    p = small_problem(1)
    full_o, full_l = A.prefill(**p.oracle_kwargs(), mode="emulate")
    o, l = A.prefill(**p.oracle_kwargs(), mode="emulate", tiles=[(0, 3, 1), (1, 0, 0)])
    np.testing.assert_array_equal(o[128:200, 3], full_o[128:200, 3])
    np.testing.assert_array_equal(l[0, 200:277], full_l[0, 200:277])
    assert np.isnan(o[0, 0, 0]) and np.isnan(l[1, 0])


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0 + 2 ** -7, -3.14159, 1e-30, 0.0])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(A.round_bf16(x.astype(np.float32).astype(np.float64)), ref)


def test_more_queries_than_keys():
    """Bottom-right alignment with Lq > Lkv: query i sits at position Lkv - Lq + i, so
    the first Lq - Lkv queries see no key (causal) and give O = 0, LSE = -FLT_MAX;
    the rest follow brute force, as do the non-causal rows (empty only where the
    block mask selects no tile)."""
    p = make_problem("tiny", seed=71, lq=(300, 50), lkv=(100, 200), hq=4, hkv=2, quant_type=1,
                     kv_layout=1, page_size=32, keep=0.6, fill="nan")
    sizes = omega_sizes(p)
    assert np.all(sizes[:, :200] == 0) and np.all(sizes[:, 200:300] > 0)
    for causal in (True, False):
        kw = {**p.oracle_kwargs(), "causal": causal}
        ob, lb = A.brute_force(**kw)
        for mode in ("exact", "emulate"):
            o, l = A.prefill(**kw, mode=mode)
            if mode == "exact":
                np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
                np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)
            if causal:
                assert np.all(o[:200] == 0.0) and np.all(l[:, :200] == NEG_FLT_MAX)
                assert np.all(l[:, 200:] > NEG_FLT_MAX)
            empty = l == NEG_FLT_MAX
            assert np.array_equal(empty, lb == NEG_FLT_MAX)
            assert np.all(o.transpose(1, 0, 2)[empty] == 0.0)
