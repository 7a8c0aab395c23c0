"""Pins of the oracle's index-list input form, probability scale and NTD query
layout ("Quant Block Sparse Attention", "Key parameters" and "Sparse indices &
PA page table").  CPU only."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import e4m3
from synth import make_problem, index_form, to_ntd

SMALL = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(129,), lkv=(383,), hq=3, hkv=3, quant_type=1, kv_layout=0, page_size=32, keep=0.3),
]


def small_problem(i, seed=21, **kw):
    return make_problem("tiny", seed=seed + i, **{**SMALL[i], **kw})


def with_index_form(p, **kw):
    idx, ln = index_form(p, **kw)
    args = p.oracle_kwargs()
    args["block_mask"] = None
    return dict(args, sparse_indices=idx, sparse_seq_len=ln)


@pytest.mark.parametrize("mode", ["exact", "emulate"])
@pytest.mark.parametrize("i", range(len(SMALL)))
def test_sorted_index_lists_equal_the_mask(mode, i):
    """Listing the switched-on tiles of the mask in ascending order selects the same
    sparse sets and visits them in the same order, so the results are identical.
    Entries that name no tile of the sequence and the unused tail are ignored."""
    p = small_problem(i)
    om, lm = A.prefill(**p.oracle_kwargs(), mode=mode)
    oi, li = A.prefill(**with_index_form(p, order="ascending", junk=True), mode=mode)
    np.testing.assert_array_equal(oi, om)
    np.testing.assert_array_equal(li, lm)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_index_form_matches_brute_force(i):
    p = small_problem(i)
    args = with_index_form(p, order="shuffled", seed=3, junk=True)
    o, l = A.prefill(**args, mode="exact")
    ob, lb = A.brute_force(**{k: v for k, v in args.items()})
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_exact_result_does_not_depend_on_list_order(i):
    p = small_problem(i)
    oa, la = A.prefill(**with_index_form(p, order="ascending", junk=False), mode="exact")
    os_, ls = A.prefill(**with_index_form(p, order="shuffled", seed=11, junk=True), mode="exact")
    np.testing.assert_allclose(os_, oa, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls, la, rtol=0, atol=1e-12)


def test_emulated_list_order_changes_only_rounding():
    """Visiting the tiles in another order changes the running maxima at which P is
    rounded, not the sparse set: the LSE is unchanged and the outputs of the two
    orders stay within two E4M3 rounding budgets of each other."""
    p = small_problem(1)
    oa, la = A.prefill(**with_index_form(p, order="ascending", junk=False), mode="emulate")
    os_, ls = A.prefill(**with_index_form(p, order="shuffled", seed=5, junk=False), mode="emulate")
    oe, _ = A.prefill(**p.oracle_kwargs(), mode="exact")
    np.testing.assert_allclose(ls, la, rtol=0, atol=1e-12)
    assert np.abs(os_ - oe).max() <= 0.1 and np.abs(oa - oe).max() <= 0.1
    assert not np.array_equal(os_, oa)


def test_empty_and_all_junk_lists():
    p = small_problem(0)
    idx, ln = index_form(p, junk=False)
    ln[0, 1, 1] = 0                            # an empty list
    idx[0, 0, 2, :3] = [-1, 7, -3]             # only entries that name no tile (Lkv = 300: 3 tiles)
    ln[0, 0, 2] = 3
    args = dict(p.oracle_kwargs(), block_mask=None, sparse_indices=idx, sparse_seq_len=ln)
    for mode in ("exact", "emulate"):
        o, l = A.prefill(**args, mode=mode)
        assert np.all(o[128:256, 1] == 0) and np.all(l[1, 128:256] == A.NEG_FLT_MAX)
        assert np.all(o[256:300, 0] == 0) and np.all(l[0, 256:300] == A.NEG_FLT_MAX)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_ntd_layout_gives_the_same_result(i):
    p = small_problem(i)
    qn, qsn = to_ntd(p)
    args = dict(p.oracle_kwargs(), q=qn, qscale=qsn, q_layout=A.NTD)
    for mode in ("exact", "emulate"):
        o0, l0 = A.prefill(**p.oracle_kwargs(), mode=mode)
        o1, l1 = A.prefill(**args, mode=mode)
        np.testing.assert_array_equal(o1, o0)
        np.testing.assert_array_equal(l1, l0)
    ob, lb = A.brute_force(**args)
    o0, l0 = A.prefill(**p.oracle_kwargs(), mode="exact")
    np.testing.assert_allclose(ob, o0, rtol=0, atol=1e-12)


def test_default_p_scale_is_256():
    p = small_problem(1)
    o0, l0 = A.prefill(**p.oracle_kwargs(), mode="emulate")
    o1, l1 = A.prefill(**p.oracle_kwargs(), mode="emulate", p_scale=256.0)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)


@pytest.mark.parametrize("p_scale, p8", [(64.0, 64.0), (300.0, 288.0), (448.0, 448.0), (1.0, 1.0), (0.3, 0.3125)])
def test_p_scale_closed_form_zero_q(p_scale, p8):
    """Q = 0: every score is 0, so P~ = 1 and P' = p_scale for every key of Omega.
    P' rounds to the E4M3 value p8 (300 -> 288: E4M3 spacing is 32 in [256, 512);
    0.3 -> 0.3125: spacing 2^-5 in [0.25, 0.5)) while the row sum keeps p_scale,
    so O = (p8 / p_scale) * mean of V^ over Omega and LSE = ln|Omega|."""
    assert e4m3.round_to_grid(np.array([p_scale]))[0] == p8
    p = small_problem(0)
    p.q[:] = 0
    o, l = A.prefill(**p.oracle_kwargs(), mode="emulate", p_scale=p_scale)
    oe, le = A.prefill(**p.oracle_kwargs(), mode="exact")
    nz = le > A.NEG_FLT_MAX
    np.testing.assert_allclose(l, le, rtol=0, atol=1e-12)
    o_nz = o.transpose(1, 0, 2)[nz]
    oe_nz = oe.transpose(1, 0, 2)[nz]
    np.testing.assert_allclose(o_nz, (p8 / p_scale) * oe_nz, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("p_scale", [16.0, 448.0])
def test_p_scale_error_bound(p_scale):
    """With scale s, rounding s*P to E4M3 moves each weight by at most half an
    E4M3 spacing: <= 2^-4 relative above 2^-6 and <= 2^-10 absolute below it
    (units of s*P).  Hence |O_emul - O_exact| <= sum_j max(2^-4 P_j, 2^-10/s) |V^_j| / l."""
    p = small_problem(0)
    oe, le = A.prefill(**p.oracle_kwargs(), mode="exact")
    om, lm = A.prefill(**p.oracle_kwargs(), mode="emulate", p_scale=p_scale)
    np.testing.assert_allclose(lm, le, rtol=0, atol=1e-12)
    kd = A._dequant_kv_sequence(p.kcache, p.kscale, p.block_table[0], 300, 0, p.page_size, p.kv_layout, False, p.kscale[0])
    vd = A._dequant_kv_sequence(p.vcache, None, p.block_table[0], 300, 0, p.page_size, p.kv_layout, False, p.vscale[0])
    for h in range(2):
        q = e4m3.decode(p.q[:, h]) * p.qscale[:, h, None].astype(np.float64)
        s = p.softmax_scale * q @ kd.T
        on = p.block_mask[0, h][np.arange(300) // 128][:, np.arange(300) // 128] != 0
        allowed = on & (np.arange(300)[None, :] <= np.arange(300)[:, None])
        s = np.where(allowed, s, -np.inf)
        mx = np.where(allowed.any(1), s.max(1), 0.0)
        pw = np.exp(s - mx[:, None])
        l = pw.sum(1)
        ok = l > 0
        bound = (np.maximum(2.0 ** -4 * pw, (2.0 ** -10 / p_scale) * allowed) @ np.abs(vd))[ok] / l[ok, None]
        assert np.all(np.abs(om[:, h] - oe[:, h])[ok] <= bound + 1e-12)
