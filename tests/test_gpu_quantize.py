"""GPU parity of the quantise-and-append step: codes, descales and both whole
caches bit for bit against the oracle (every slot outside the appended ones
must keep its old bytes), then the full chain quantise -> append -> prefill
against the oracle chain."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import quantize as Qz
from synth import make_problem, append_inputs
from parity_util import compare

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


CASES = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(64, 256, 1), lkv=(250, 256, 700), hq=4, hkv=1, quant_type=1, kv_layout=0, page_size=64,
         keep=0.7),
    dict(lq=(0, 129, 1000), lkv=(40, 383, 1500), hq=16, hkv=2, quant_type=0, kv_layout=1, page_size=32,
         keep=0.4),
]


def run_gpu_quantize(p, a, pow2):
    """Quantise/append on cuda:0 into device copies of the problem's caches."""
    import block_sparse_fp8_amd as bsa
    d = p.to_device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q_in = t(a["q"]).to(torch.bfloat16)
    k_in = t(a["k"]).to(torch.bfloat16)
    v_in = t(a["v"]).to(torch.bfloat16)
    kscale_cache = d["kscale"] if p.quant_type == 1 else None
    qo, qs = bsa.bsa_fp8_quantize_append(
        q_in, k_in, v_in, d["cu_seqlens_q"], d["seqlens_kv"], d["block_table"], t(a["kscale"]),
        t(a["vscale"]), p.quant_type, p.page_size, kcache=d["kcache"], vcache=d["vcache"],
        kscale_cache=kscale_cache, kv_layout=p.kv_layout, scale_mode=1 if pow2 else 0)
    torch.cuda.synchronize()
    u8 = lambda x: x.view(torch.uint8).cpu().numpy()  # noqa: E731
    return (u8(qo), qs.cpu().numpy(), u8(d["kcache"]), u8(d["vcache"]),
            None if kscale_cache is None else kscale_cache.cpu().numpy(), d)


def oracle_quantize(p, a, pow2):
    return Qz.quantize_append(a["q"], a["k"], a["v"], p.cu_seqlens_q, p.seqlens_kv, p.block_table,
                              a["kscale"], a["vscale"], p.quant_type, p.page_size, p.kv_layout,
                              p.kcache, p.vcache, p.kscale if p.quant_type == 1 else None,
                              pow2=pow2)


def assert_same(got, want):
    names = ("q codes", "qscale", "kcache", "vcache", "kscale cache")
    for name, g, w in zip(names, got, want):
        if w is None:
            continue
        if g.dtype == np.float32:
            np.testing.assert_array_equal(g.view(np.uint32), np.asarray(w, np.float32).view(np.uint32),
                                          err_msg=name)
        else:
            np.testing.assert_array_equal(g, w, err_msg=name)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_quantize_append_bitwise(i, pow2):
    p = make_problem("tiny", seed=400 + i, **CASES[i])
    a = append_inputs(p, seed=40 + i)
    say(f"[gpu] quantize/append case {i} pow2={pow2} lq={p.cfg.lq} lkv={p.cfg.lkv}")
    got = run_gpu_quantize(p, a, pow2)
    assert_same(got[:5], oracle_quantize(p, a, pow2))


@pytest.mark.parametrize("pow2", [False, True])
def test_power_of_two_input_scaling(pow2):
    """Inputs times 2^5 (exact in bfloat16) leave every computed-descale code
    unchanged and multiply those descales by 32 (amax/448 and its power-of-two
    rounding both commute with the factor); all-zero rows keep descale 1.
    Checked on Q and, with quant type 1, on the appended K slots and their
    cached descales; the oracle is not involved."""
    p = make_problem("tiny", seed=401, **CASES[1])  # quant type 1
    a = append_inputs(p, seed=41)
    say(f"[gpu] quantize power-of-two input scaling pow2={pow2}")
    q1, qs1, kc1, _, ks1, _ = run_gpu_quantize(p, a, pow2)
    a2 = dict(a, q=a["q"] * np.float32(32.0), k=a["k"] * np.float32(32.0))
    q2, qs2, kc2, _, ks2, _ = run_gpu_quantize(p, a2, pow2)
    np.testing.assert_array_equal(q2, q1)
    zero_q = np.abs(a["q"]).max(axis=2) == 0
    np.testing.assert_array_equal(qs2, np.where(zero_q, qs1, qs1 * np.float32(32.0)))
    np.testing.assert_array_equal(kc2, kc1)
    changed = ks1 != np.asarray(p.kscale, np.float32)  # the appended slots (old ones are kept)
    assert changed.sum() > 0
    ratio = ks2[changed] / ks1[changed]
    assert np.all((ratio == np.float32(32.0)) | (ks1[changed] == np.float32(1.0)))


def test_quantize_q_only_and_append_only():
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=420, **CASES[1])
    a = append_inputs(p, seed=42)
    d = p.to_device("cuda")
    want = oracle_quantize(p, a, False)
    say("[gpu] quantize Q only")
    qo, qs = bsa.bsa_fp8_quantize_append(
        torch.from_numpy(a["q"]).cuda().to(torch.bfloat16), None, None, None, None, None, None, None,
        p.quant_type, p.page_size, kcache=None, vcache=None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qo.view(torch.uint8).cpu().numpy(), want[0])
    np.testing.assert_array_equal(qs.cpu().numpy(), want[1])
    say("[gpu] append only")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    bsa.bsa_fp8_quantize_append(
        None, t(a["k"]).to(torch.bfloat16), t(a["v"]).to(torch.bfloat16), d["cu_seqlens_q"],
        d["seqlens_kv"], d["block_table"], t(a["kscale"]), t(a["vscale"]), p.quant_type,
        p.page_size, kcache=d["kcache"], vcache=d["vcache"], kscale_cache=d["kscale"],
        kv_layout=p.kv_layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d["kcache"].view(torch.uint8).cpu().numpy(), want[2])
    np.testing.assert_array_equal(d["vcache"].view(torch.uint8).cpu().numpy(), want[3])
    np.testing.assert_array_equal(d["kscale"].cpu().numpy(), want[4])


# Given descales on both sides of the range [2^-80, 2^100] in which the kernel
# forms quotients from one reciprocal per row (outside it, it divides per value),
# and Q rows whose computed descale amax/448 falls on either side of 2^-80.
EDGE_DESCALES = [2.0 ** -90, float(np.nextafter(np.float32(2.0 ** -80), np.float32(0))), 2.0 ** -80,
                 2.0 ** 100, float(np.nextafter(np.float32(2.0 ** 100), np.float32(np.inf))), 2.0 ** 110]


@pytest.mark.parametrize("quant_type", [0, 1])
@pytest.mark.parametrize("dsc", EDGE_DESCALES)
def test_quantize_descale_range_edges(dsc, quant_type):
    p = make_problem("tiny", seed=450, **dict(CASES[0], quant_type=quant_type))
    a = append_inputs(p, seed=45, spread=False)
    rng = np.random.default_rng(46)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()  # noqa: E731
    # Q rows scaled by 2^e: computed descales from ~2^-109 to ~2^-60 straddle 2^-80
    e = rng.choice([-100, -92, -88, -84, -81, -80, -79, -76, -70, -60], size=a["q"].shape[:2])
    a["q"] = bf(a["q"] * np.exp2(e)[..., None])
    # K and V rows ~ 64 * N(0,1) * dsc, so their quotients by the given descale span the E4M3 grid
    a["k"] = bf(a["k"] * 64.0 * dsc)
    a["v"] = bf(a["v"] * 64.0 * dsc)
    a["kscale"] = np.array([dsc], np.float32)
    a["vscale"] = np.full(a["vscale"].shape, dsc, np.float32)
    say(f"[gpu] quantize descale edge {dsc:.3g} quant {quant_type}")
    got = run_gpu_quantize(p, a, False)
    assert_same(got[:5], oracle_quantize(p, a, False))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["sparse16k", "varlen", "dense8k"])
def test_full_size_bitwise(name):
    p = make_problem(name)
    a = append_inputs(p, seed=7)
    say(f"[gpu] full {name} quantize/append")
    got = run_gpu_quantize(p, a, False)
    assert_same(got[:5], oracle_quantize(p, a, False))


@pytest.mark.parametrize("i", [1, 3])
def test_chain_quantize_append_prefill(i):
    """GPU chain (quantise, append, prefill) against the oracle chain."""
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=430 + i, **CASES[i])
    a = append_inputs(p, seed=43 + i, spread=False)
    say(f"[gpu] chain case {i}")
    qc, qs, kc, vc, ks, d = run_gpu_quantize(p, a, False)
    vs = torch.from_numpy(a["vscale"]).cuda()
    ksc = d["kscale"] if p.quant_type == 1 else torch.from_numpy(a["kscale"]).cuda()
    q_dev = torch.from_numpy(qc).cuda().view(torch.float8_e4m3fn)
    qs_dev = torch.from_numpy(qs).cuda()
    o, l = bsa.bsa_fp8_prefill(q_dev, d["kcache"], d["vcache"], qs_dev, ksc, vs,
                               d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"],
                               d["block_mask"], p.quant_type, p.page_size,
                               max_seqlen_q=p.max_seqlen_q, kv_layout=p.kv_layout,
                               causal=p.causal, softmax_scale=p.softmax_scale)
    torch.cuda.synchronize()
    go = o.float().double().cpu().numpy()
    gl = l.double().cpu().numpy()
    oq, oqs, okc, ovc, oks = oracle_quantize(p, a, False)
    kw = p.oracle_kwargs()
    kw.update(q=oq, qscale=oqs, kcache=okc, vcache=ovc, vscale=a["vscale"],
              kscale=oks if p.quant_type == 1 else a["kscale"])
    eo, el = A.prefill(**kw, mode="emulate")
    xo, _ = A.prefill(**kw, mode="exact")
    say(f"[gpu]   ok {compare(go, gl, eo, el, xo)}")
