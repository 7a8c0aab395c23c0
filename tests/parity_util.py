"""Helpers shared by the GPU tests: run the HIP path through the C ABI binding and
compare with the oracle at the tolerances of the precision table."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PREC = json.load(open(os.path.join(GOLDEN, "precision_table.json")))
O_RTOL = PREC["attention_out"]["rtol"]
O_ATOL = PREC["attention_out"]["atol"]
L_RTOL = PREC["softmax_lse"]["rtol"]
L_ATOL = PREC["softmax_lse"]["atol"]
MAX_FRAC = PREC["max_outlier_fraction"]
EXACT_MAX_ABS = PREC["exact_oracle_max_abs_diff"]["value"]
NEG_FLT_MAX = np.float32(-3.4028234663852886e38)


def run_gpu(problem, mask=True, causal=None, out=None, lse=None):
    """Run bsa_fp8_prefill on cuda:0 and return (out float64 [T,Hq,128], lse float64 [Hq,T])."""
    import torch
    import block_sparse_fp8_amd as bsa
    d = problem.to_device("cuda")
    o, l = bsa.bsa_fp8_prefill(
        d["q"], d["kcache"], d["vcache"], d["qscale"], d["kscale"], d["vscale"],
        d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"], d["block_mask"] if mask else None,
        problem.quant_type, problem.page_size, max_seqlen_q=problem.max_seqlen_q,
        kv_layout=problem.kv_layout, causal=problem.causal if causal is None else causal,
        softmax_scale=problem.softmax_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().double().cpu().numpy(), l.double().cpu().numpy()


def tile_rows(problem, tiles):
    """Boolean selectors [T,Hq] of the rows covered by (b,h,m) tiles."""
    T, Hq, _ = problem.q.shape
    sel = np.zeros((T, Hq), dtype=bool)
    for b, h, m in tiles:
        t0 = int(problem.cu_seqlens_q[b])
        lq = int(problem.cu_seqlens_q[b + 1]) - t0
        sel[t0 + m * 128: t0 + min(m * 128 + 128, lq), h] = True
    return sel


def stats_of(got_o, got_l, emu_o, emu_l, exact_o, sel=None):
    """The quantities the acceptance rule looks at, without asserting."""
    if sel is None:
        sel = np.ones(got_o.shape[:2], dtype=bool)
    go, eo, xo = got_o[sel], emu_o[sel], exact_o[sel]
    gl, el = got_l.T[sel], emu_l.T[sel]
    bad_o = np.abs(go - eo) > O_ATOL + O_RTOL * np.abs(eo)
    bad_l = np.abs(gl - el) > L_ATOL + L_RTOL * np.abs(el)
    return dict(n=int(go.size), frac_o=float(bad_o.mean()) if bad_o.size else 0.0,
                frac_lse=float(bad_l.mean()) if bad_l.size else 0.0,
                max_abs_vs_emulate=float(np.abs(go - eo).max()) if go.size else 0.0,
                max_abs_vs_exact=float(np.abs(go - xo).max()) if go.size else 0.0,
                finite=bool(np.all(np.isfinite(go)) and np.all(np.isfinite(gl))))


def compare(got_o, got_l, emu_o, emu_l, exact_o, sel=None, exact_bound=None):
    """Assert the acceptance rule; return a dict of statistics.

    O vs the P-emulating oracle: |d| <= atol + rtol*|ref| for all but at most
    0.5% of the elements; LSE vs the oracle likewise with its own tolerances;
    O vs the exact oracle: max |d| <= 0.1.  Rows with an empty sparse set must
    be exactly 0 / -FLT_MAX.  exact_bound replaces the 0.1 of the exact check
    (for P-scales other than 256, whose rounding error is the method's own).
    """
    bound = EXACT_MAX_ABS if exact_bound is None else exact_bound
    if sel is None:
        sel = np.ones(got_o.shape[:2], dtype=bool)
    go, eo, xo = got_o[sel], emu_o[sel], exact_o[sel]
    gl, el = got_l.T[sel], emu_l.T[sel]
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    bad_o = np.abs(go - eo) > O_ATOL + O_RTOL * np.abs(eo)
    bad_l = np.abs(gl - el) > L_ATOL + L_RTOL * np.abs(el)
    frac_o = bad_o.mean() if bad_o.size else 0.0
    frac_l = bad_l.mean() if bad_l.size else 0.0
    max_exact = np.abs(go - xo).max() if go.size else 0.0
    empty = el == NEG_FLT_MAX
    stats = dict(n=int(go.size), frac_o=float(frac_o), frac_lse=float(frac_l),
                 max_abs_vs_emulate=float(np.abs(go - eo).max()) if go.size else 0.0,
                 max_abs_vs_exact=float(max_exact), empty_rows=int(empty.sum()))
    assert frac_o <= MAX_FRAC, stats
    assert frac_l <= MAX_FRAC, stats
    assert max_exact <= bound, stats
    assert np.all(gl[empty] == NEG_FLT_MAX), stats
    assert np.all(go[empty] == 0.0), stats
    return stats


def run_gpu_ex(problem, mask=True, causal=None, q_layout=0, p_scale=None, index_form=None,
               schedule=None, qk_precision=0):
    """Run bsa_fp8_prefill_ex on cuda:0: optional NTD queries, P-scale, index
    lists (sparse_indices, sparse_seq_len) instead of the mask, and a task
    order.  Returns (out float64 [T,Hq,128], lse float64 [Hq,T])."""
    import torch
    import block_sparse_fp8_amd as bsa
    from synth import to_ntd
    d = problem.to_device("cuda")
    q, qs = d["q"], d["qscale"]
    if q_layout == 1:
        qn, qsn = to_ntd(problem)
        q = torch.from_numpy(qn).cuda().view(torch.float8_e4m3fn)
        qs = torch.from_numpy(qsn).cuda()
    si = sl = None
    if index_form is not None:
        si = torch.from_numpy(np.ascontiguousarray(index_form[0])).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(index_form[1])).cuda()
    sched = None if schedule is None else torch.from_numpy(np.ascontiguousarray(schedule)).cuda()
    o, l = bsa.bsa_fp8_prefill_ex(
        q, d["kcache"], d["vcache"], qs, d["kscale"], d["vscale"],
        d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"],
        d["block_mask"] if (mask and index_form is None) else None,
        problem.quant_type, problem.page_size, max_seqlen_q=problem.max_seqlen_q,
        kv_layout=problem.kv_layout, causal=problem.causal if causal is None else causal,
        softmax_scale=problem.softmax_scale, q_layout=q_layout, p_scale=p_scale,
        sparse_indices=si, sparse_seq_len=sl, schedule=sched, qk_precision=qk_precision)
    torch.cuda.synchronize()
    return o.float().double().cpu().numpy(), l.double().cpu().numpy()


def run_schedule(problem, mask=True, index_form=None, causal=None):
    """bsa_fp8_schedule on cuda:0 for the problem's lengths and sparsity;
    returns the task order as int32 numpy."""
    import torch
    import block_sparse_fp8_amd as bsa
    d = problem.to_device("cuda")
    si = sl = None
    if index_form is not None:
        si = torch.from_numpy(np.ascontiguousarray(index_form[0])).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(index_form[1])).cuda()
    s = bsa.bsa_fp8_schedule(
        d["cu_seqlens_q"], d["seqlens_kv"],
        d["block_mask"] if (mask and index_form is None) else None,
        num_heads_q=problem.q.shape[1], max_seqlen_q=problem.max_seqlen_q,
        causal=problem.causal if causal is None else causal, sparse_indices=si,
        sparse_seq_len=sl)
    torch.cuda.synchronize()
    return s.cpu().numpy()
