"""Pins of the quantise-and-append oracle (oracle/quantize.py): hand-encoded
codes from the E4M3 format definition, properties that follow from the
descale rule, the reconstruction error bound, the placement of appended rows
(checked slot by slot), and an end-to-end check through the attention
oracle."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import e4m3
from oracle import quantize as Qz
from synth import make_problem, append_inputs


def bf16(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_hand_encoded_row():
    # amax 448 -> descale exactly 1; codes from the format (sign, 4-bit exponent
    # with bias 7, 3-bit mantissa): 448 = 1.75*2^8 -> 0 1111 110 = 0x7E;
    # -224 = -1.75*2^7 -> 1 1110 110 = 0xF6; 1.5 = 1.5*2^0 -> 0 0111 100 = 0x3C;
    # 2^-9 (smallest subnormal) -> 0x01; 0 -> 0x00; 0.75 = 1.5*2^-1 -> 0 0110 100 = 0x34.
    x = np.zeros(128, dtype=np.float32)
    x[:6] = [448.0, -224.0, 1.5, 2.0 ** -9, 0.0, 0.75]
    codes, d = Qz.quantize_rows(x[None])
    assert d[0] == np.float32(1.0)
    assert list(codes[0, :6]) == [0x7E, 0xF6, 0x3C, 0x01, 0x00, 0x34]
    assert np.all(codes[0, 6:] == 0)


def test_descale_of_a_half_row():
    # amax 224 -> descale 0.5 (exact), every value doubles before encoding
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0], x[0, 1] = -224.0, 3.0
    codes, d = Qz.quantize_rows(x)
    assert d[0] == np.float32(0.5)
    assert codes[0, 0] == 0xFE and codes[0, 1] == 0x4C   # -448; 6 = 1.5*2^2 -> 0 1001 100


def test_zero_row():
    codes, d = Qz.quantize_rows(np.zeros((3, 128), dtype=np.float32))
    assert np.all(d == 1.0) and np.all(codes == 0)
    codes, d = Qz.quantize_rows(np.zeros((1, 128), dtype=np.float32), pow2=True)
    assert np.all(d == 1.0)


def random_rows(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= np.exp2(rng.uniform(-30, 30, size=(n, 1))).astype(np.float32)
    return bf16(x)


@pytest.mark.parametrize("seed", range(3))
def test_amax_lands_on_448(seed):
    """With d = fp32(amax/448), amax/d is within a few float32 ulps of 448,
    so the largest element of every row encodes to +-448."""
    x = random_rows(4000, seed)
    codes, d = Qz.quantize_rows(x)
    j = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(x.shape[0]), j]
    assert np.all((top & 0x7F) == 0x7E)


@pytest.mark.parametrize("seed", range(3))
def test_pow2_descale_properties(seed):
    x = random_rows(4000, seed + 10)
    amax = np.max(np.abs(x), axis=1).astype(np.float64)
    _, d = Qz.quantize_rows(x, pow2=True)
    m, _ = np.frexp(d.astype(np.float64))
    assert np.all(m == 0.5)                                  # a power of two
    assert np.all(d >= amax / 448 * (1 - 2 ** -23))          # covers amax (up to the fp32 division)
    assert np.all(d < 2 * amax / 448 * (1 + 2 ** -23))       # the smallest such power
    codes, _ = Qz.quantize_rows(x, pow2=True)
    assert np.all(np.abs(e4m3.decode(codes)) <= 448)


@pytest.mark.parametrize("pow2", [False, True])
def test_reconstruction_error_bound(pow2):
    """|decode(code)*d - x| <= d * (half an E4M3 step at |x/d|) + fp32 slack."""
    x = random_rows(3000, 7)
    codes, d = Qz.quantize_rows(x, pow2)
    y = x.astype(np.float64) / d[:, None]
    rec = e4m3.decode(codes)
    ay = np.abs(y)
    # E4M3 step at |y|: 2^(floor(log2|y|) - 3) for normals (|y| >= 2^-6), 2^-9 below
    step = np.where(ay >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(rec - y)
    assert np.all(err <= step / 2 * (1 + 1e-6) + ay * 2.0 ** -23)


def test_power_of_two_scaling_invariance():
    x = random_rows(500, 3)
    x = x / np.float32(2.0 ** 40)                 # keep 2^k multiples inside the normal range
    c0, d0 = Qz.quantize_rows(x)
    for k in (-5, 7, 19):
        ck, dk = Qz.quantize_rows(x * np.float32(2.0 ** k))
        np.testing.assert_array_equal(ck, c0)
        np.testing.assert_array_equal(dk, d0 * np.float32(2.0 ** k))


def test_given_descale_saturates():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :3] = [10.0, -1e6, 0.5]
    codes = Qz.encode_with(x, np.array([1.0 / 64], dtype=np.float32))
    # 640 saturates to 448 (0x7E), -6.4e7 to -448 (0xFE), 32 = 1.0*2^5 -> 0 1100 000 = 0x60
    assert list(codes[0, :3]) == [0x7E, 0xFE, 0x60]


CASES = [
    dict(lq=(300,), lkv=(300,), hq=2, hkv=1, quant_type=0, kv_layout=0, page_size=64, keep=0.5),
    dict(lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1, page_size=32, keep=0.5),
    dict(lq=(64, 256, 1), lkv=(250, 256, 700), hq=4, hkv=1, quant_type=1, kv_layout=0, page_size=64,
         keep=0.7),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_append_places_rows_slot_by_slot(i):
    p = make_problem("tiny", seed=300 + i, **CASES[i])
    a = append_inputs(p, seed=i)
    ksc = p.kscale if p.quant_type == 1 else None
    qc, qs, kc, vc, ks = Qz.quantize_append(
        a["q"], a["k"], a["v"], p.cu_seqlens_q, p.seqlens_kv, p.block_table, a["kscale"],
        a["vscale"], p.quant_type, p.page_size, p.kv_layout, p.kcache, p.vcache, ksc)
    assert qc.shape == a["q"].shape and qs.shape == a["q"].shape[:2]
    touched = np.zeros(kc.shape[:3], dtype=bool)
    for b in range(len(p.seqlens_kv)):
        t0, t1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        for t in range(t0, t1):
            pos = int(p.seqlens_kv[b]) - (t1 - t0) + (t - t0)
            page = int(p.block_table[b, pos // p.page_size])
            slot = pos % p.page_size
            for g in range(p.cfg.hkv):
                idx = (page, slot, g) if p.kv_layout == 0 else (page, g, slot)
                touched[idx] = True
                kd = ks[idx] if p.quant_type == 1 else a["kscale"][0]
                vd = a["vscale"][g] if p.quant_type == 1 else a["vscale"][0]
                # each stored row reconstructs its input within half an E4M3 step
                for cache, src, d in ((kc, a["k"], kd), (vc, a["v"], vd)):
                    rec = e4m3.decode(cache[idx]) * float(d)
                    x = src[t, g].astype(np.float64)
                    ok = np.abs(rec - x) <= np.maximum(np.abs(x) * 2.0 ** -4, float(d) * 2.0 ** -10) * 1.0001
                    sat = np.abs(x) >= 448 * float(d)
                    assert np.all(ok | sat), (b, t, g)
                    assert np.all(np.abs(rec[sat]) == 448 * float(d))
    # every other slot (and its descale) is untouched
    np.testing.assert_array_equal(kc[~touched], p.kcache[~touched])
    np.testing.assert_array_equal(vc[~touched], p.vcache[~touched])
    if p.quant_type == 1:
        np.testing.assert_array_equal(ks[~touched], p.kscale[~touched])


def test_end_to_end_through_attention():
    """Quantise the chunk, append it, run the attention oracle on the result:
    close to exact attention on the bfloat16 inputs (the keys outside the
    chunk keep the problem's own cache)."""
    cfg = dict(lq=(256,), lkv=(256,), hq=4, hkv=2, quant_type=1, kv_layout=0, page_size=64, keep=1.0)
    p = make_problem("tiny", seed=310, **cfg)
    a = append_inputs(p, seed=3, spread=False)
    qc, qs, kc, vc, ks = Qz.quantize_append(
        a["q"], a["k"], a["v"], p.cu_seqlens_q, p.seqlens_kv, p.block_table, a["kscale"],
        a["vscale"], p.quant_type, p.page_size, p.kv_layout, p.kcache, p.vcache, p.kscale)
    kw = p.oracle_kwargs()
    kw.update(q=qc, qscale=qs, kcache=kc, vcache=vc, kscale=ks, vscale=a["vscale"])
    o, lse = A.prefill(**kw, mode="exact")
    # reference on the unquantised values (Lq = Lkv: the whole cache is the chunk)
    q = a["q"].astype(np.float64)
    k = a["k"].astype(np.float64)
    v = a["v"].astype(np.float64)
    T = q.shape[0]
    ref = np.zeros_like(o)
    for h in range(4):
        g = h // 2
        sc = (q[:, h] @ k[:, g].T) / np.sqrt(128.0)
        sc[np.triu(np.ones((T, T), dtype=bool), 1)] = -np.inf
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        ref[:, h] = (w / w.sum(axis=1, keepdims=True)) @ v[:, g]
    # V descales 0.010..0.015 saturate V at 4.5..6.7; N(0,1) data almost never reaches that
    # E4M3 keeps 3 mantissa bits (a relative half-step of 2^-4 per value), so
    # the error is of that order per element: measured rms 0.008, max 0.107
    # (early queries that attend to a handful of keys).  A misplaced row or a
    # wrong descale gives errors of order 1.
    err = np.abs(o - ref)
    assert np.sqrt((err ** 2).mean()) < 0.02
    assert err.max() < 0.25
