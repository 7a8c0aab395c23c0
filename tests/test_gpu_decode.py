"""GPU parity of FP8 sparse decode against the fp64 oracle.

The kernel's arithmetic fixes the bound: dequantised K and V are exact in
bfloat16 (E4M3 codes times power-of-two descales), Q is bfloat16, products
accumulate in fp32, and two roundings remain, each by at most 2^-8 relative
(bfloat16 keeps 8 significant bits): every probability to bfloat16 before
P.V, and the output to bfloat16.  So for every element
|O_gpu - O| <= 2^-8 (A + |O|) with A = sum_j P_j |v_j| (the
oracle's weighted magnitude), plus a 5% and 1e-6 margin for the fp32
accumulation and exp2 steps; no element may exceed it.  LSE involves no
bfloat16 step: rtol 5e-3 / atol 2.5e-5 as for the prefill.  Rows with no
valid index must be exactly 0 / -FLT_MAX."""
import numpy as np
import pytest

from oracle import decode as D
from synth import make_decode_problem
from parity_util import L_RTOL, L_ATOL, MAX_FRAC

pytestmark = pytest.mark.gpu

NEG_FLT_MAX = np.float32(-3.4028234663852886e38)


def say(msg):
    print(msg, flush=True)


def run_gpu(p, num_splits=None, workspace=None):
    """num_splits None: the plain entry point; else the split-list one."""
    import torch
    import block_sparse_fp8_amd as bsa
    d = p.to_device("cuda")
    if num_splits is None:
        o, l = bsa.bsa_fp8_sparse_decode(d["q"], d["kv_cache"], d["indices"], softmax_scale=p.softmax_scale)
    else:
        o, l = bsa.bsa_fp8_sparse_decode_ex(d["q"], d["kv_cache"], d["indices"], num_splits=num_splits,
                                            workspace=workspace, softmax_scale=p.softmax_scale)
    torch.cuda.synchronize()
    return o.float().double().cpu().numpy(), l.double().cpu().numpy()


def compare(go, gl, eo, el, ea, pairs=None):
    """ea: the oracle's weighted magnitude A; pairs: (b, s) query tokens to
    compare (default: all)."""
    if pairs is not None:
        go = np.stack([go[b, s] for b, s in pairs])
        eo = np.stack([eo[b, s] for b, s in pairs])
        ea = np.stack([ea[b, s] for b, s in pairs])
        gl = np.stack([gl[b, :, s] for b, s in pairs])
        el = np.stack([el[b, :, s] for b, s in pairs])
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    err = np.abs(go - eo)
    bound = 2.0 ** -8 * 1.05 * (ea + np.abs(eo)) + 1e-6
    bad_l = np.abs(gl - el) > L_ATOL + L_RTOL * np.abs(el)
    empty = el == NEG_FLT_MAX
    stats = dict(n=int(go.size), over_bound=int((err > bound).sum()),
                 worst_ratio=float((err / bound).max()), frac_lse=float(bad_l.mean()),
                 max_abs=float(err.max()), empty=int(empty.sum()))
    assert stats["over_bound"] == 0, stats
    assert stats["frac_lse"] <= MAX_FRAC, stats
    assert np.all(gl[empty] == NEG_FLT_MAX), stats
    return stats


SMALL = [
    dict(lkv=(300, 1000), s_q=2, h_q=64, topk=200, ragged=True),
    dict(lkv=(70,), s_q=1, h_q=128, topk=64, page_size=32),
    dict(lkv=(1500, 40, 333), s_q=3, h_q=64, topk=77, ragged=True),
    dict(lkv=(20, 500), s_q=1, h_q=64, topk=5),                # top-k below one block
    dict(lkv=(2048,), s_q=2, h_q=128, topk=2048, page_size=64),
    dict(lkv=(900, 350), s_q=1, h_q=192, topk=300, ragged=True),   # three 64-head groups
    dict(lkv=(20, 3), s_q=2, h_q=64, topk=1),                  # a single entry per list
    dict(lkv=(700,), s_q=2, h_q=256, topk=96, page_size=32),   # two 128-head workgroups per token
]


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small_vs_oracle(i):
    p = make_decode_problem("decode_tiny", seed=500 + i, **SMALL[i])
    say(f"[gpu] decode small{i} lkv={p.cfg.lkv} s_q={p.cfg.s_q} h_q={p.cfg.h_q} topk={p.cfg.topk}")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")


@pytest.mark.parametrize("frac", [1.0, 0.5])
def test_descales_not_powers_of_two(frac):
    """Descales that are not powers of two take the fp32-product path (the
    power-of-two ones a single scaled conversion).  Multiplying a descale by
    1.5 keeps code * descale exact in bfloat16 (4 + 2 significant bits), so
    the bound above still holds; frac 0.5 changes half the (token, tile)
    descales, so lanes of one wave take different paths."""
    p = make_decode_problem("decode_tiny", seed=520, **SMALL[0])
    rng = np.random.default_rng(521)
    sc = p.kv_cache[..., 512:528].copy().view(np.float32)       # [pages, page_size, 4]
    pick = rng.random(sc.shape) < frac
    with np.errstate(over="ignore", invalid="ignore"):  # unused slots hold random bytes
        sc[pick] *= np.float32(1.5)
    p.kv_cache[..., 512:528] = sc.view(np.uint8)
    say(f"[gpu] decode descales x1.5 on {frac:.0%} of tiles")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")
    go2, gl2 = run_gpu(p, num_splits=3)
    compare(go2, gl2, eo, el, ea)


def test_zero_softmax_scale_is_the_mean_of_the_selected_rows():
    """softmax_scale = 0: every valid entry weighs 1 (P = 2^0 is exact in bfloat16), so O
    is the mean of the named rows' dequantised values (a repeated entry counts twice) and
    LSE = log(count).  The closed form decodes the row bytes with torch's E4M3 type, not
    with the oracle."""
    import torch
    from parity_util import NEG_FLT_MAX
    p = make_decode_problem("decode_tiny", seed=530, **SMALL[2])
    p.softmax_scale = 0.0
    say("[gpu] decode softmax scale 0, plain and 3 parts")
    got = [run_gpu(p), run_gpu(p, num_splits=3)]
    rows = p.kv_cache.reshape(-1, p.kv_cache.shape[-1])
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :512])).view(torch.float8_e4m3fn).double().numpy()
    B, s_q, h_q, _ = p.q.shape
    for b in range(B):
        for s in range(s_q):
            idx = p.indices[b, s].astype(np.int64)
            idx = idx[(idx >= 0) & (idx < rows.shape[0])]
            for go, gl in got:
                if idx.size == 0:
                    assert np.all(go[b, s] == 0.0) and np.all(gl[b, :, s] == NEG_FLT_MAX)
                    continue
                scales = np.ascontiguousarray(rows[idx, 512:528]).view(np.float32).astype(np.float64)
                v = codes[idx] * np.repeat(scales, 128, axis=1)               # [n, 512]
                mean = v.mean(axis=0)
                tol = 2.0 ** -8 * np.abs(mean) + 2.0 ** -14 * np.abs(v).max()
                assert np.all(np.abs(go[b, s] - mean[None, :]) <= tol[None, :]), (b, s)
                np.testing.assert_allclose(gl[b, :, s], np.log(idx.size), rtol=1e-5, atol=1e-6)

@pytest.mark.parametrize("factor", [4.0, 16.0, 64.0])
def test_peaked_softmax(factor):
    """Q times a power of two (exact in bfloat16) spreads the scores over
    tens to hundreds of binades: each head's softmax is dominated by a few
    tokens, its reference maximum moves on many blocks (by more than 2^8 at a
    time), and most P round to bfloat16 subnormals or zero.  The bound above
    does not depend on the spread.  The split-list form is checked too."""
    p = make_decode_problem("decode_tiny", seed=530, **SMALL[4])
    p.q = (p.q * np.float32(factor)).astype(np.float32)
    say(f"[gpu] decode peaked softmax, Q x{factor:g}")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")
    go2, gl2 = run_gpu(p, num_splits=5)
    say(f"[gpu]   split ok {compare(go2, gl2, eo, el, ea)}")


def n_rows(p):
    return p.kv_cache.shape[0] * p.kv_cache.shape[1]


def test_row_permutation_invariance():
    """Moving every cache row to another place and renaming the list entries
    to match (entries that name no row left as they are) gives bit-identical
    results: an index is a cache row id and nothing else."""
    p = make_decode_problem("decode_tiny", seed=531, **SMALL[2])
    say("[gpu] decode row permutation")
    o1, l1 = run_gpu(p)
    rows = n_rows(p)
    perm = np.random.default_rng(532).permutation(rows)
    flat = p.kv_cache.reshape(rows, -1)
    moved = np.empty_like(flat)
    moved[perm] = flat
    p.kv_cache = moved.reshape(p.kv_cache.shape)
    valid = (p.indices >= 0) & (p.indices < rows)
    p.indices = np.where(valid, perm[np.clip(p.indices, 0, rows - 1)], p.indices).astype(np.int32)
    o2, l2 = run_gpu(p)
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(l2, l1)


def test_empty_lists_and_sequences():
    p = make_decode_problem("decode_tiny", seed=510, lkv=(300, 0, 90), s_q=2, h_q=64, topk=40)
    p.indices[0, 1, :] = -1                          # nothing selected
    p.indices[2, 0, :20] = n_rows(p) + np.arange(20)   # entries that name no row
    p.indices[2, 0, 20:] = -7 - np.arange(20)
    say("[gpu] decode empty lists / empty sequence")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    compare(go, gl, eo, el, ea)
    for b, s in ((0, 1), (1, 0), (1, 1), (2, 0)):
        assert np.all(go[b, s] == 0.0) and np.all(gl[b, :, s] == NEG_FLT_MAX)


def test_rows_of_any_page():
    """Entries are cache rows, not positions of the query's own sequence: each
    list takes rows of every sequence's pages, in the page-block index *
    page_size + slot encoding, with rows of physical page 0 and the last row
    of the cache among them."""
    p = make_decode_problem("decode_tiny", seed=514, lkv=(200, 333), s_q=2, h_q=64, topk=96)
    rows = np.array(sorted({p.row_of(b, j) for b in range(2) for j in range(p.cfg.lkv[b])}))
    rng = np.random.default_rng(14)
    for b in range(2):
        for s in range(2):
            p.indices[b, s] = rng.choice(rows, size=96, replace=False)
    p.indices[0, 0, :3] = [rows.min(), rows.max(), -1]
    say("[gpu] decode rows of any page")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")


def test_unused_entries_with_nan_in_row_zero():
    """Entries that name no row are staged from row 0; with NaN codes,
    descales and RoPE values there, the result must still be finite and equal
    the oracle's, which never reads an unnamed row."""
    p = make_decode_problem("decode_tiny", seed=515, lkv=(300, 1000), s_q=2, h_q=64, topk=200, ragged=True)
    ps = p.kv_cache.shape[1]
    p.indices[(p.indices >= 0) & (p.indices < ps)] = -1    # nothing names page 0
    p.kv_cache[0, :, :512] = 0x7F                          # E4M3 NaN
    p.kv_cache[0, :, 512:] = 0xFF                          # NaN descales and bfloat16 NaN
    assert (p.indices == -1).any()
    say("[gpu] decode unused entries, NaN in row 0")
    for splits in (None, 3):
        go, gl = run_gpu(p, num_splits=splits)
        eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
        say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")


def test_repeated_entries_count_twice():
    p = make_decode_problem("decode_tiny", seed=511, lkv=(400,), s_q=1, h_q=64, topk=50)
    p.indices[0, 0, 25:] = p.indices[0, 0, :25]       # every token listed twice
    say("[gpu] decode repeated entries")
    go, gl = run_gpu(p)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    compare(go, gl, eo, el, ea)


def test_unselected_rows_never_read():
    a = make_decode_problem("decode_tiny", seed=512, fill="random")
    b = make_decode_problem("decode_tiny", seed=512, fill="nan")
    say("[gpu] decode NaN in unselected rows")
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_deterministic():
    p = make_decode_problem("decode_tiny", seed=513)
    say("[gpu] decode determinism")
    o1, l1 = run_gpu(p)
    o2, l2 = run_gpu(p)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def sampled_oracle(p, go, gl, pairs):
    eo = np.zeros_like(go)
    ea = np.zeros_like(go)
    el = np.zeros_like(gl)
    for b, s in pairs:
        one = D.sparse_decode(p.q[b:b + 1, s:s + 1], p.kv_cache, p.indices[b:b + 1, s:s + 1],
                              p.softmax_scale, with_abs=True)
        eo[b, s] = one[0][0, 0]
        el[b, :, s] = one[1][0, :, 0]
        ea[b, s] = one[2][0, 0]
    return eo, el, ea


@pytest.mark.timeout(600)
def test_full_size_sampled():
    p = make_decode_problem("decode_b128")
    say("[gpu] decode full size B=128 s_q=2 h_q=128 topk=2048 (16 sampled query tokens)")
    go, gl = run_gpu(p)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    rng = np.random.default_rng(3)
    pairs = sorted({(int(rng.integers(0, 128)), int(rng.integers(0, 2))) for _ in range(16)} | {(0, 0), (127, 1)})
    eo, el, ea = sampled_oracle(p, go, gl, pairs)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea, pairs)}")


# ---- split-list path: each list cut into parts, partial results merged ----------

@pytest.mark.parametrize("splits", [2, 3, 7, "auto"])
@pytest.mark.parametrize("i", [0, 2, 3, 4, 5])
def test_split_small_vs_oracle(i, splits):
    """Parts of 1+ blocks, parts that select nothing (top-k 5 is one block, so
    every part after the first is empty) and ragged lists."""
    p = make_decode_problem("decode_tiny", seed=500 + i, **SMALL[i])
    say(f"[gpu] split decode small{i} splits={splits} lkv={p.cfg.lkv} topk={p.cfg.topk}")
    go, gl = run_gpu(p, num_splits=splits)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")


def test_split_one_equals_plain_bitwise():
    p = make_decode_problem("decode_tiny", seed=520, lkv=(700, 1200), s_q=2, h_q=128, topk=500, ragged=True)
    say("[gpu] split decode num_splits=1 vs plain entry point")
    a = run_gpu(p)
    b = run_gpu(p, num_splits=1)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_split_empty_lists_and_sequences():
    p = make_decode_problem("decode_tiny", seed=521, lkv=(300, 0, 90), s_q=2, h_q=64, topk=100)
    p.indices[0, 1, :] = -1
    p.indices[2, 0, :] = n_rows(p) + np.arange(100)   # entries that name no row
    p.indices[0, 0, 32:] = -1                      # only the first part selects anything
    say("[gpu] split decode empty lists / empty sequence")
    go, gl = run_gpu(p, num_splits=4)
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    compare(go, gl, eo, el, ea)
    for b, s in ((0, 1), (1, 0), (1, 1), (2, 0)):
        assert np.all(go[b, s] == 0.0) and np.all(gl[b, :, s] == NEG_FLT_MAX)


def test_split_lists_longer_than_one_workgroup():
    """10000 entries: above the 8192 one workgroup holds, so at least two parts."""
    import block_sparse_fp8_amd as bsa
    p = make_decode_problem("decode_tiny", seed=522, lkv=(12000,), s_q=1, h_q=64, topk=10000, ragged=True)
    n = bsa.bsa_fp8_sparse_decode_num_splits(1, 1, 64, 10000)
    assert n >= 2
    say(f"[gpu] split decode topk=10000 splits={n} and 2")
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    for splits in (n, 2):
        go, gl = run_gpu(p, num_splits=splits)
        say(f"[gpu]   ok {compare(go, gl, eo, el, ea)}")


def test_split_reused_workspace():
    """One workspace for two calls of different sizes; the second call must not
    see the first one's partial results."""
    import torch
    import block_sparse_fp8_amd as bsa
    a = make_decode_problem("decode_tiny", seed=523, lkv=(2000, 900), s_q=2, h_q=128, topk=1000)
    b = make_decode_problem("decode_tiny", seed=524, lkv=(50,), s_q=1, h_q=64, topk=40)
    ws = torch.empty(bsa.bsa_fp8_sparse_decode_workspace_bytes(2, 2, 128, 5), dtype=torch.uint8, device="cuda")
    say("[gpu] split decode reused workspace")
    for p in (a, b):
        go, gl = run_gpu(p, num_splits=5, workspace=ws)
        eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
        compare(go, gl, eo, el, ea)


@pytest.mark.timeout(600)
def test_split_full_size_long_lists_sampled():
    import block_sparse_fp8_amd as bsa
    p = make_decode_problem("decode_long16k")
    n = bsa.bsa_fp8_sparse_decode_num_splits(4, 2, 128, 16384)
    say(f"[gpu] split decode full size B=4 s_q=2 h_q=128 topk=16384 splits={n} (all 8 query tokens)")
    go, gl = run_gpu(p, num_splits=n)
    pairs = [(b, s) for b in range(4) for s in range(2)]
    eo, el, ea = sampled_oracle(p, go, gl, pairs)
    say(f"[gpu]   ok {compare(go, gl, eo, el, ea, pairs)}")
