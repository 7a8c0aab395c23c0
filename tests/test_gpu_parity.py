"""GPU parity: the HIP kernel through the C ABI versus the fp64 oracle.

Small shapes are compared on every output element; the five workload
configurations at full size are compared on seeded samples of Q tiles (the
launch is the full problem, exactly as the benchmark times it), plus
properties that hold for every output element.
"""
import numpy as np
import torch
import pytest

from oracle import attention as A
from synth import make_problem
from synth.workloads import sample_q_tiles
from parity_util import run_gpu, compare, tile_rows, NEG_FLT_MAX

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def check(problem, tiles=None, mask=True, causal=None, label=""):
    say(f"[gpu] {label} cfg={problem.cfg.name} lq={problem.cfg.lq} lkv={problem.cfg.lkv} "
        f"hq={problem.cfg.hq} hkv={problem.cfg.hkv} quant={problem.quant_type} "
        f"layout={problem.kv_layout} ps={problem.page_size} mask={mask} tiles={None if tiles is None else len(tiles)}")
    go, gl = run_gpu(problem, mask=mask, causal=causal)
    kw = problem.oracle_kwargs()
    if not mask:
        kw["block_mask"] = None
    if causal is not None:
        kw["causal"] = causal
    eo, el = A.prefill(**kw, mode="emulate", tiles=tiles)
    xo, _ = A.prefill(**kw, mode="exact", tiles=tiles)
    sel = None if tiles is None else tile_rows(problem, tiles)
    stats = compare(go, gl, eo, el, xo, sel)
    say(f"[gpu]   ok {stats}")
    return go, gl


SMALL = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(129,), lkv=(383,), hq=3, hkv=3, quant_type=1, kv_layout=0, page_size=32, keep=0.3),
    dict(lq=(64, 256, 1), lkv=(250, 256, 700), hq=4, hkv=1, quant_type=0, kv_layout=1, page_size=64,
         keep=0.7),
    dict(lq=(1000,), lkv=(1500,), hq=16, hkv=1, quant_type=1, kv_layout=0, page_size=64, keep=0.4),
]


def test_tiny_config_all_elements():
    check(make_problem("tiny"), label="tiny")


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("page_size", [32, 64])
@pytest.mark.parametrize("quant", [0, 1])
def test_layout_page_quant_matrix(layout, page_size, quant):
    p = make_problem("tiny", kv_layout=layout, page_size=page_size, quant_type=quant)
    check(p, label=f"matrix L{layout} P{page_size} Q{quant}")


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small_shapes_all_elements(i):
    check(make_problem("tiny", seed=50 + i, **SMALL[i]), label=f"small{i}")


def test_skip_ratio_zero_and_null_mask():
    p = make_problem("tiny", seed=9, **{**SMALL[1], "keep": 1.0})
    p.block_mask[:] = 1
    o1, l1 = check(p, label="all-ones mask")
    o2, l2 = check(p, mask=False, label="NULL mask")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_non_causal():
    check(make_problem("tiny", seed=11, **SMALL[0]), causal=False, label="non-causal")
    check(make_problem("tiny", seed=12, **SMALL[1]), causal=False, label="non-causal varlen")


def test_empty_rows_exact():
    p = make_problem("tiny", seed=13, **SMALL[1])
    p.block_mask[1, 2, 0, :] = 0               # whole Q tile empty
    p.block_mask[0, 1, 0, :] = 0               # only a future tile: early rows empty
    p.block_mask[0, 1, 0, 2] = 1
    go, gl = check(p, label="empty rows")
    t0 = int(p.cu_seqlens_q[1])
    assert np.all(go[t0:t0 + 77, 2] == 0.0)
    assert np.all(gl[2, t0:t0 + 77] == NEG_FLT_MAX)
    pos = 390 - 200 + np.arange(128)
    assert np.all(gl[1, :128][pos < 256] == NEG_FLT_MAX)
    assert np.all(gl[1, :128][pos >= 256] > NEG_FLT_MAX)


def test_nan_in_unused_slots_and_spare_pages():
    cfg = SMALL[4]
    a = make_problem("tiny", seed=14, fill="zero", **cfg)
    b = make_problem("tiny", seed=14, fill="nan", **cfg)
    say("[gpu] nan-fill pair")
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_nan_in_skipped_pages():
    cfg = dict(lq=(256,), lkv=(1024,), hq=4, hkv=2, quant_type=1, kv_layout=0, page_size=64, keep=1.0)
    a = make_problem("tiny", seed=15, identity_pages=True, **cfg)
    b = make_problem("tiny", seed=15, identity_pages=True, **cfg)
    for p in (a, b):
        p.block_mask[:, :, :, 2] = 0           # KV tile 2 (keys 256..383) off everywhere
    b.kcache[4:6] = 0x7F                       # its pages hold NaN
    b.vcache[4:6] = 0x7F
    b.kscale[4:6] = np.nan
    say("[gpu] nan skipped pages")
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    assert np.all(np.isfinite(ob))
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_page_permutation_invariance():
    a = make_problem("tiny", seed=16, identity_pages=True, **SMALL[3])
    b = make_problem("tiny", seed=16, identity_pages=False, **SMALL[3])
    say("[gpu] page permutation")
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_zero_q_closed_form():
    p = make_problem("tiny", seed=17, **SMALL[1])
    p.q[:] = 0
    say("[gpu] Q=0 closed form")
    go, gl = run_gpu(p)
    eo, el = A.prefill(**p.oracle_kwargs(), mode="exact")
    ok = el > NEG_FLT_MAX
    # LSE = ln|Omega| exactly up to fp32 rounding; O = mean of V^ over Omega
    np.testing.assert_allclose(gl[ok], el[ok], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(go, eo, rtol=2 ** -7, atol=1e-4)


@pytest.mark.parametrize("i", [0, 1])
def test_descale_power_of_two_invariance(i):
    """Q descales times 2^-7 with K descales times 2^7 leave every score
    unchanged, and V descales times 8 scale O by 8: power-of-two factors are
    exact in fp32 and bf16, so LSE must be bit-identical and O exactly 8x
    (quant 0: per-tensor K descale; quant 1: per token and head)."""
    p = make_problem("tiny", seed=19, **SMALL[i])
    say(f"[gpu] descale power-of-two invariance, quant {p.quant_type}")
    o1, l1 = run_gpu(p)
    p.qscale = (p.qscale * np.float32(2.0 ** -7)).astype(np.float32)
    p.kscale = (p.kscale * np.float32(2.0 ** 7)).astype(np.float32)
    p.vscale = (p.vscale * np.float32(8.0)).astype(np.float32)
    o2, l2 = run_gpu(p)
    np.testing.assert_array_equal(l2, l1)
    np.testing.assert_array_equal(o2, 8.0 * o1)


def test_causal_equals_non_causal_below_the_diagonal():
    """With every selected tile strictly below the diagonal (Lq = Lkv), no
    selected key is past any query, so causal and non-causal runs visit the
    same tiles in the same order with nothing to mask: bit-identical results
    (and a mask that selects the diagonal tile must differ)."""
    p = make_problem("tiny", seed=20, lq=(600, 256), lkv=(600, 256), hq=2, hkv=1, quant_type=1,
                     kv_layout=0, page_size=64, keep=0.7)
    bm = p.block_mask
    mt, nt = bm.shape[2], bm.shape[3]
    below = np.tril(np.ones((mt, nt), dtype=np.uint8), k=-1)
    bm[:] = bm * below
    say("[gpu] causal vs non-causal, tiles below the diagonal only")
    oc, lc = run_gpu(p, causal=True)
    on, ln = run_gpu(p, causal=False)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)
    bm[:, :, 1, 1] = 1  # the diagonal tile of Q tile 1: now the band mask matters
    oc, lc = run_gpu(p, causal=True)
    on, ln = run_gpu(p, causal=False)
    assert not np.array_equal(lc, ln)


def test_deterministic():
    p = make_problem("tiny", seed=18, **SMALL[4])
    say("[gpu] determinism")
    o1, l1 = run_gpu(p)
    o2, l2 = run_gpu(p)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_widest_mask_and_extra_rows_ignored():
    """A mask of the widest accepted shape (4096 KV tiles) with three extra
    Q-tile rows, random bits everywhere outside the tight shape: tiles past a
    sequence's KV length and rows past its queries select nothing, so the
    result is the tight mask's, bit for bit."""
    import dataclasses
    p = make_problem("tiny", seed=19, **SMALL[1])
    B, Hq, mt, mkv = p.block_mask.shape
    rng = np.random.default_rng(19)
    wide = rng.integers(0, 2, size=(B, Hq, mt + 3, 4096), dtype=np.uint8)
    wide[:, :, :mt, :mkv] = p.block_mask
    q = dataclasses.replace(p, block_mask=wide)
    go, gl = check(p, label="tight mask")
    say("[gpu] widest mask")
    wo, wl = run_gpu(q)
    np.testing.assert_array_equal(go, wo)
    np.testing.assert_array_equal(gl, wl)


def test_sequences_without_queries():
    """Batch entries with no query tokens (with and without cached keys) next to
    ordinary ones: they produce no work and do not disturb the others."""
    p = make_problem("tiny", seed=20, lq=(0, 150, 0, 33), lkv=(300, 260, 0, 33), hq=4, hkv=2,
                     quant_type=1, kv_layout=1, page_size=32, keep=0.6)
    check(p, label="sequences without queries")
    check(p, causal=False, label="sequences without queries, non-causal")


def test_lse_not_requested_leaves_output_unchanged():
    """lse = NULL: the epilogue skips the LSE store; O is the same bit for bit."""
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=81, **SMALL[1])
    say("[gpu] prefill without lse")
    d = p.to_device("cuda")
    args = (d["q"], d["kcache"], d["vcache"], d["qscale"], d["kscale"], d["vscale"], d["cu_seqlens_q"],
            d["block_table"], d["seqlens_kv"], d["block_mask"], p.quant_type, p.page_size)
    kw = dict(max_seqlen_q=p.max_seqlen_q, kv_layout=p.kv_layout, causal=p.causal,
              softmax_scale=p.softmax_scale)
    o1, l1 = bsa.bsa_fp8_prefill(*args, **kw)
    o2, l2 = bsa.bsa_fp8_prefill(*args, **kw, return_lse=False)
    assert l2 is None
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_zero_softmax_scale_is_the_mean_of_the_selected_values():
    """softmax_scale = 0: every selected key weighs the same, P' = 256 is exact in E4M3, so
    O is the mean of the dequantised V rows of each query's keys and LSE = log(count).
    The closed form is computed here from the codes (torch's E4M3 decoding), not by the oracle."""
    p = make_problem("tiny", seed=82, **SMALL[1])
    p.softmax_scale = 0.0
    go, gl = check(p, label="softmax scale 0")
    T, Hq, _ = p.q.shape
    Hkv = p.vcache.shape[1] if p.kv_layout == 1 else p.vcache.shape[2]
    codes = torch.from_numpy(np.ascontiguousarray(p.vcache)).view(torch.float8_e4m3fn).double().numpy()
    vs = np.asarray(p.vscale, dtype=np.float64)
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lq, lkv = t1 - t0, int(p.seqlens_kv[b])
        j = np.arange(lkv)
        page, slot = p.block_table[b, j // p.page_size], j % p.page_size
        for h in range(Hq):
            g = h // (Hq // Hkv)
            v = (codes[page, g, slot] if p.kv_layout == 1 else codes[page, slot, g])
            v = v * (vs[g] if vs.size > 1 else vs[0])                     # [lkv, 128]
            for t in range(lq):
                on = (p.block_mask[b, h, t // 128, j // 128] != 0) & (j <= lkv - lq + t)
                n = int(on.sum())
                if n == 0:
                    assert np.all(go[t0 + t, h] == 0.0) and gl[h, t0 + t] == NEG_FLT_MAX
                    continue
                mean = v[on].mean(axis=0)
                tol = 2.0 ** -8 * np.abs(mean) + 2.0 ** -12 * np.abs(v[on]).max()
                assert np.all(np.abs(go[t0 + t, h] - mean) <= tol), (b, h, t)
                assert abs(gl[h, t0 + t] - np.log(n)) <= 1e-5 * max(1.0, np.log(n)), (b, h, t)

def test_more_queries_than_keys():
    """Lq > Lkv: query i sits at position Lkv - Lq + i, so (causal) the first Lq - Lkv
    queries see no key, including whole waves inside a visited tile."""
    p = make_problem("tiny", seed=72, lq=(300, 50), lkv=(100, 200), hq=4, hkv=2, quant_type=1,
                     kv_layout=1, page_size=32, keep=0.6, fill="nan")
    go, gl = check(p, label="more queries than keys")
    assert np.all(go[:200] == 0.0) and np.all(gl[:, :200] == NEG_FLT_MAX)
    check(p, causal=False, label="more queries than keys, non-causal")


FULL = [("dense8k", 40, ()), ("sparse16k", 48, ()), ("varlen", 48, ((3, 5, 17), (0, 0, 0))),
        ("long128k", 64, ((0, 0, 0), (0, 31, 1023), (0, 7, 1)))]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,count,must", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(name, count, must):
    p = make_problem(name)
    tiles = sample_q_tiles(p, count, seed=1, must_include=must)
    go, gl = check(p, tiles=tiles, label=f"full {name}")
    # properties of every element: finite, LSE finite or the empty marker
    assert np.all(np.isfinite(go))
    assert np.all(np.isfinite(gl))
    if name == "varlen":
        t0 = int(p.cu_seqlens_q[3])
        rows = slice(t0 + 17 * 128, t0 + 18 * 128)
        assert np.all(go[rows, 5] == 0.0)
        assert np.all(gl[5, rows] == NEG_FLT_MAX)
