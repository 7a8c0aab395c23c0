"""GPU parity of the extended entry point and the scheduling pre-pass: the
index-list form, the NTD query layout, the P-scale, and task orders written on
the device, each against the oracle (and, where the arithmetic is the same,
bit for bit against the plain entry point)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import schedule as S
from synth import make_problem, index_form, topk_index_form, to_ntd
from synth.workloads import sample_q_tiles
from parity_util import run_gpu, run_gpu_ex, run_schedule, compare, tile_rows, NEG_FLT_MAX

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


SMALL = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(64, 256, 1), lkv=(250, 256, 700), hq=4, hkv=1, quant_type=0, kv_layout=1, page_size=64,
         keep=0.7),
    dict(lq=(1000,), lkv=(1500,), hq=16, hkv=1, quant_type=1, kv_layout=0, page_size=64, keep=0.4),
    dict(lq=(300, 50), lkv=(100, 200), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32,
         keep=0.6),  # more queries than keys: the first 200 rows see no key
]


def oracle_pair(p, tiles=None, index=None, p_scale=None, causal=None, mask=True):
    kw = p.oracle_kwargs()
    if index is not None or not mask:
        kw["block_mask"] = None
    if index is not None:
        kw["sparse_indices"], kw["sparse_seq_len"] = index
    if causal is not None:
        kw["causal"] = causal
    eo, el = A.prefill(**kw, mode="emulate", tiles=tiles, p_scale=p_scale)
    xo, _ = A.prefill(**kw, mode="exact", tiles=tiles)
    return eo, el, xo


def oracle_schedule(p, index=None, mask=True, causal=None):
    kw = {}
    if index is not None:
        kw = dict(sparse_indices=index[0], sparse_seq_len=index[1])
    elif mask:
        kw = dict(block_mask=p.block_mask)
    c = S.task_costs(p.cu_seqlens_q, p.seqlens_kv, p.q.shape[1], p.max_seqlen_q,
                     p.causal if causal is None else causal, **kw)
    return S.schedule(c, p.q.shape[1], p.max_seqlen_q)


# ---- index-list form -------------------------------------------------------------

@pytest.mark.parametrize("i", range(len(SMALL)))
def test_ascending_list_equals_mask_bitwise(i):
    """Ascending lists with junk entries visit the same tiles in the same order
    as the mask, so every output bit matches the mask form."""
    p = make_problem("tiny", seed=60 + i, **SMALL[i])
    say(f"[gpu] ascending list vs mask small{i}")
    mo, ml = run_gpu(p)
    lo, ll = run_gpu_ex(p, index_form=index_form(p, "ascending", seed=i, junk=True))
    np.testing.assert_array_equal(lo, mo)
    np.testing.assert_array_equal(ll, ml)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_shuffled_list_vs_oracle(i):
    p = make_problem("tiny", seed=70 + i, **SMALL[i])
    idx = index_form(p, "shuffled", seed=100 + i, junk=True)
    say(f"[gpu] shuffled list small{i}")
    go, gl = run_gpu_ex(p, index_form=idx)
    eo, el, xo = oracle_pair(p, index=idx)
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo)}")


@pytest.mark.parametrize("causal", [True, False])
def test_topk_list_vs_oracle(causal):
    """Lists that do not come from a mask, shorter than the number of KV tiles,
    with tiles above the causal range."""
    p = make_problem("tiny", seed=80, **SMALL[3])
    idx = topk_index_form(p, 5, seed=81)
    say(f"[gpu] top-k list causal={causal}")
    go, gl = run_gpu_ex(p, index_form=idx, causal=causal)
    eo, el, xo = oracle_pair(p, index=idx, causal=causal)
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo)}")


def test_list_empty_and_junk_rows():
    p = make_problem("tiny", seed=82, **SMALL[1])
    idx, slen = index_form(p, "shuffled", seed=83, junk=True)
    slen[1, 2, 0] = 0                       # empty list
    idx[0, 1, 1, :] = -1                    # only junk
    idx[0, 3, 0, :] = 99
    slen[0, 0, 1] = -4                      # negative length = empty
    row = idx.shape[3]                      # longer than the row: clipped to the row
    idx[1, 0, 0, :] = np.array([-1, 3, 0, 7, -2, 5, 8, 9][:row], dtype=np.int32)
    slen[1, 0, 0] = 10 ** 6
    say("[gpu] empty / junk lists")
    go, gl = run_gpu_ex(p, index_form=(idx, slen))
    eo, el, xo = oracle_pair(p, index=(idx, slen))
    compare(go, gl, eo, el, xo)
    t0 = int(p.cu_seqlens_q[1])
    assert np.all(go[t0:t0 + 77, 2] == 0.0) and np.all(gl[2, t0:t0 + 77] == NEG_FLT_MAX)
    assert np.all(go[128:200, 1] == 0.0) and np.all(gl[1, 128:200] == NEG_FLT_MAX)
    assert np.all(go[0:128, 3] == 0.0) and np.all(gl[3, 0:128] == NEG_FLT_MAX)
    assert np.all(gl[0, 128:200] == NEG_FLT_MAX)


# ---- NTD queries and the P-scale --------------------------------------------------

@pytest.mark.parametrize("i", [1, 3])
def test_ntd_layout(i):
    p = make_problem("tiny", seed=90 + i, **SMALL[i])
    say(f"[gpu] NTD small{i}")
    to, tl = run_gpu(p)
    no, nl = run_gpu_ex(p, q_layout=1)
    np.testing.assert_array_equal(no, to)
    np.testing.assert_array_equal(nl, tl)
    qn, qsn = to_ntd(p)
    kw = p.oracle_kwargs()
    kw.update(q=qn, qscale=qsn)
    eo, el = A.prefill(**kw, mode="emulate", q_layout=A.NTD)
    xo, _ = A.prefill(**kw, mode="exact", q_layout=A.NTD)
    compare(no, nl, eo, el, xo)


# The 0.1 bound against the exact oracle is that of P-scale 256, where the
# row maximum's probability lands exactly on the E4M3 grid.  Other scales put it
# between grid points (300: a step of 32 around it), and the emulating oracle
# itself then moves further from the exact result; the kernel is held to that
# distance plus a margin of twice the largest kernel-vs-emulation difference
# seen at 256 (0.008).
EXACT_MARGIN = 0.02


def exact_bound_for(eo, xo):
    return max(0.1, float(np.nanmax(np.abs(eo - xo))) + EXACT_MARGIN)


@pytest.mark.parametrize("ps", [64.0, 300.0, 448.0, 1.0, 0.3])
def test_p_scale_vs_oracle(ps):
    p = make_problem("tiny", seed=95, **SMALL[1])
    say(f"[gpu] p_scale={ps}")
    go, gl = run_gpu_ex(p, p_scale=ps)
    eo, el, xo = oracle_pair(p, p_scale=ps)
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo, exact_bound=exact_bound_for(eo, xo))}")


def test_p_scale_default_is_256_bitwise():
    p = make_problem("tiny", seed=96, **SMALL[0])
    say("[gpu] p_scale default")
    ao, al = run_gpu(p)
    for ps in (None, 0.0, 256.0):
        bo, bl = run_gpu_ex(p, p_scale=ps)
        np.testing.assert_array_equal(bo, ao)
        np.testing.assert_array_equal(bl, al)


def test_p_scale_changes_rounding_only():
    """A different P-scale moves P across other E4M3 rounding points, and
    nothing else: the result against the exact oracle stays within bound."""
    p = make_problem("tiny", seed=97, **SMALL[3])
    say("[gpu] p_scale rounding")
    ao, _ = run_gpu_ex(p, p_scale=256.0)
    bo, _ = run_gpu_ex(p, p_scale=300.0)
    assert np.any(ao != bo)
    eo, _, xo = oracle_pair(p, p_scale=300.0)
    assert np.abs(bo - xo).max() <= exact_bound_for(eo, xo)


# ---- scheduling pre-pass ----------------------------------------------------------

def test_schedule_small_forms_match_oracle():
    for i, cfg in enumerate(SMALL):
        p = make_problem("tiny", seed=110 + i, **cfg)
        idx = index_form(p, "shuffled", seed=i, junk=True)
        for label, kw in (("mask", {}), ("dense", dict(mask=False)), ("list", dict(index_form=idx)),
                          ("non-causal", dict(causal=False))):
            say(f"[gpu] schedule small{i} {label}")
            got = run_schedule(p, **kw)
            want = oracle_schedule(p, index=kw.get("index_form"), mask=kw.get("mask", True),
                                   causal=kw.get("causal"))
            np.testing.assert_array_equal(got, want)


def test_schedule_many_blocks_and_cost_cap():
    # 3 * 24 * 32 = 2304 tasks (three rank blocks); then a single sequence long
    # enough for costs above the 1023 cap.
    cfg = dict(lq=(4096, 1000, 3000), lkv=(4096, 5000, 3100), hq=24, hkv=8, quant_type=0,
               kv_layout=0, page_size=64, keep=0.5)
    p = make_problem("tiny", seed=120, **cfg)
    say("[gpu] schedule 2304 tasks")
    np.testing.assert_array_equal(run_schedule(p), oracle_schedule(p))
    idx = topk_index_form(p, 9, seed=121)
    np.testing.assert_array_equal(run_schedule(p, index_form=idx), oracle_schedule(p, index=idx))
    long = dict(lq=(140000,), lkv=(140000,), hq=1, hkv=1, quant_type=0, kv_layout=0,
                page_size=64, keep=1.0)
    q = make_problem("tiny", seed=122, **long)
    say("[gpu] schedule with costs above the cap")
    want = oracle_schedule(q, mask=False)
    assert S.task_costs(q.cu_seqlens_q, q.seqlens_kv, 1, q.max_seqlen_q, True).max() > 1023
    np.testing.assert_array_equal(run_schedule(q, mask=False), want)


@pytest.mark.parametrize("i", [1, 3])
def test_prefill_with_schedule_bitwise(i):
    """The order changes which tasks run first, never a result."""
    p = make_problem("tiny", seed=130 + i, **SMALL[i])
    idx = index_form(p, "shuffled", seed=i, junk=True)
    say(f"[gpu] prefill with schedule small{i}")
    for kw in (dict(), dict(index_form=idx), dict(mask=False)):
        ao, al = run_gpu_ex(p, **kw)
        sched = run_schedule(p, **kw)
        bo, bl = run_gpu_ex(p, schedule=sched, **kw)
        np.testing.assert_array_equal(bo, ao)
        np.testing.assert_array_equal(bl, al)


# ---- full-size workloads ------------------------------------------------------------

FULL = [("sparse16k", 32, ()), ("varlen", 32, ((3, 5, 17), (0, 0, 0)))]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,count,must", FULL, ids=[f[0] for f in FULL])
def test_full_size_shuffled_list_with_schedule(name, count, must):
    p = make_problem(name)
    idx = index_form(p, "shuffled", seed=7, junk=True)
    tiles = sample_q_tiles(p, count, seed=2, must_include=must)
    say(f"[gpu] full {name}: schedule, shuffled lists, {len(tiles)} sampled Q tiles")
    sched = run_schedule(p, index_form=idx)
    np.testing.assert_array_equal(sched, oracle_schedule(p, index=idx))
    go, gl = run_gpu_ex(p, index_form=idx, schedule=sched)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    eo, el, xo = oracle_pair(p, tiles=tiles, index=idx)
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo, tile_rows(p, tiles))}")


@pytest.mark.timeout(600)
def test_full_size_long_schedule():
    p = make_problem("long128k")
    say("[gpu] full long128k schedule")
    np.testing.assert_array_equal(run_schedule(p), oracle_schedule(p))


def test_all_options_together():
    """NTD queries, shuffled index lists with junk, P-scale 64 and a device
    schedule in one call, against the oracle with the same options."""
    p = make_problem("tiny", seed=140, **SMALL[3])
    idx = index_form(p, "shuffled", seed=141, junk=True)
    say("[gpu] NTD + index lists + p_scale 64 + schedule")
    sched = run_schedule(p, index_form=idx)
    go, gl = run_gpu_ex(p, q_layout=1, p_scale=64.0, index_form=idx, schedule=sched)
    qn, qsn = to_ntd(p)
    kw = p.oracle_kwargs()
    kw.update(q=qn, qscale=qsn, block_mask=None, sparse_indices=idx[0], sparse_seq_len=idx[1])
    eo, el = A.prefill(**kw, mode="emulate", q_layout=A.NTD, p_scale=64.0)
    xo, _ = A.prefill(**kw, mode="exact", q_layout=A.NTD)
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo)}")
    # same bits as the TND call without a schedule
    to, tl = run_gpu_ex(p, p_scale=64.0, index_form=idx)
    np.testing.assert_array_equal(go, to)
    np.testing.assert_array_equal(gl, tl)
