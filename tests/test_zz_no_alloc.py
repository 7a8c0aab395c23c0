"""bsa_fp8_sparse_decode_noalloc: the split-list decode with its partial
results in the library's static scratch, for callers that cannot allocate.

Checked through the C ABI against bsa_fp8_sparse_decode_ex (the same kernels
with a caller workspace) bit for bit, on two calls in a row where the second
is smaller (the scratch keeps the first call's contents), and with the
library's own part count against the fp64 oracle."""
import numpy as np
import pytest

from oracle import decode as D
from synth import make_decode_problem
from parity_util import L_RTOL, L_ATOL

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_both(p, splits):
    import torch
    import block_sparse_fp8_amd as bsa
    d = p.to_device("cuda")
    B, s_q, h_q, _ = p.q.shape
    ws = torch.empty(max(1, bsa.bsa_fp8_sparse_decode_workspace_bytes(B, s_q, h_q, splits)), dtype=torch.uint8,
                     device="cuda")
    o1, l1 = bsa.bsa_fp8_sparse_decode_ex(d["q"], d["kv_cache"], d["indices"], num_splits=splits, workspace=ws,
                                          softmax_scale=p.softmax_scale)
    o2 = torch.full((B, s_q, h_q, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    l2 = torch.full((B, h_q, s_q), float("nan"), dtype=torch.float32, device="cuda")
    bsa.bsa_fp8_sparse_decode_noalloc(d["q"], d["kv_cache"], d["indices"], o2, l2, num_splits=splits,
                                      softmax_scale=p.softmax_scale)
    torch.cuda.synchronize()
    return (o1.view(torch.int16).cpu().numpy(), l1.cpu().numpy()), (o2.view(torch.int16).cpu().numpy(),
                                                                    l2.cpu().numpy())


def test_noalloc_equals_workspace_entry_two_calls():
    big = make_decode_problem("decode_tiny", seed=700, lkv=(3000, 5000), s_q=2, h_q=128, topk=2500, ragged=True)
    small = make_decode_problem("decode_tiny", seed=701, lkv=(300,), s_q=1, h_q=64, topk=100, ragged=True)
    for p, splits in ((big, 9), (small, 3)):
        say(f"[gpu] noalloc decode lkv={p.cfg.lkv} h_q={p.cfg.h_q} topk={p.cfg.topk} splits={splits}")
        (o1, l1), (o2, l2) = run_both(p, splits)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_noalloc_library_part_count_vs_oracle():
    import torch
    import block_sparse_fp8_amd as bsa
    p = make_decode_problem("decode_tiny", seed=702, lkv=(900, 2000), s_q=2, h_q=64, topk=700, ragged=True)
    d = p.to_device("cuda")
    B, s_q, h_q, _ = p.q.shape
    out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device="cuda")
    say("[gpu] noalloc decode, library part count")
    bsa.bsa_fp8_sparse_decode_noalloc(d["q"], d["kv_cache"], d["indices"], out, lse, softmax_scale=p.softmax_scale)
    torch.cuda.synchronize()
    go = out.float().double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    eo, el, ea = D.sparse_decode(**p.oracle_kwargs(), with_abs=True)
    # the decode's element bound: two bfloat16 roundings (P and O), fp32 sums
    bound = 2.0 ** -8 * 1.05 * (ea + np.abs(eo)) + 1e-6
    assert np.all(np.abs(go - eo) <= bound)
    ok = el > -3e38
    assert np.all(np.abs(gl[ok] - el[ok]) <= L_ATOL + L_RTOL * np.abs(el[ok]))
    assert np.all(gl[~ok] == np.float32(-3.4028234663852886e38))
