"""The entry points inside captured HIP graphs.

None of them allocates, synchronises or reads device memory on the host, so
a serving loop can capture them.  Each test captures calls on static buffers,
then replays the graph several times; before each replay new inputs are
copied into those buffers, eagerly and with a synchronisation, and every
replay's outputs must equal, bit for bit, an eager call on the same inputs
(the kernels are deterministic).  The eager results themselves are checked
against the oracle by the other GPU tests.
"""
import numpy as np
import pytest
import torch

from synth import make_problem, make_decode_problem, append_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 4


def say(msg):
    print(msg, flush=True)


def capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("split", [False, True])
def test_decode_graph_replays(split):
    import block_sparse_fp8_amd as bsa
    p = make_decode_problem("decode_tiny", seed=600, lkv=(900, 1500), s_q=2, h_q=128, topk=700, ragged=True)
    d = p.to_device("cuda")
    B, s_q, h_q, _ = p.q.shape
    out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device="cuda")
    splits = 5
    ws = torch.empty(bsa.bsa_fp8_sparse_decode_workspace_bytes(B, s_q, h_q, splits), dtype=torch.uint8,
                     device="cuda")

    def call(o, l):
        if split:
            bsa.bsa_fp8_sparse_decode_ex(d["q"], d["kv_cache"], d["indices"], num_splits=splits, workspace=ws,
                                         softmax_scale=p.softmax_scale, out=o, lse=l)
        else:
            bsa.bsa_fp8_sparse_decode(d["q"], d["kv_cache"], d["indices"], softmax_scale=p.softmax_scale,
                                      out=o, lse=l)

    say(f"[gpu] graph decode split={split}")
    g = capture(lambda: call(out, lse))
    rng = np.random.default_rng(601)
    for r in range(REPLAYS):
        q_new = torch.from_numpy(rng.standard_normal(p.q.shape, dtype=np.float32)).to(torch.bfloat16)
        idx_new = torch.from_numpy(np.ascontiguousarray(rng.permuted(p.indices, axis=2)))
        d["q"].copy_(q_new)
        d["indices"].copy_(idx_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo = torch.empty_like(out)
        el = torch.empty_like(lse)
        call(eo, el)
        torch.cuda.synchronize()
        assert same(out, eo) and same(lse, el), f"replay {r}"
    say("[gpu]   ok")


def test_prefill_graph_replays():
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=610, lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1,
                     page_size=32, keep=0.5)
    d = p.to_device("cuda")
    T, Hq, D = p.q.shape
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")

    def call(o, l):
        bsa.bsa_fp8_prefill(d["q"], d["kcache"], d["vcache"], d["qscale"], d["kscale"], d["vscale"],
                            d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"], d["block_mask"],
                            p.quant_type, p.page_size, max_seqlen_q=p.max_seqlen_q, kv_layout=p.kv_layout,
                            causal=p.causal, softmax_scale=p.softmax_scale, out=o, lse=l)

    say("[gpu] graph prefill")
    g = capture(lambda: call(out, lse))
    rng = np.random.default_rng(611)
    for r in range(REPLAYS):
        # new E4M3 codes (finite ones only: 0x7F / 0xFF are NaN) and a new mask
        codes = rng.integers(0, 0x7F, size=p.q.shape, dtype=np.uint8) | (rng.integers(0, 2, size=p.q.shape,
                                                                                    dtype=np.uint8) << 7)
        d["q"].view(torch.uint8).copy_(torch.from_numpy(codes))
        d["block_mask"].copy_(torch.from_numpy(rng.integers(0, 2, size=p.block_mask.shape, dtype=np.uint8)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo = torch.empty_like(out)
        el = torch.empty_like(lse)
        call(eo, el)
        torch.cuda.synchronize()
        assert same(out, eo) and same(lse, el), f"replay {r}"
    say("[gpu]   ok")


def test_schedule_and_prefill_graph_replays():
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=620, lq=(64, 256, 1), lkv=(250, 256, 700), hq=8, hkv=1, quant_type=0,
                     kv_layout=1, page_size=64, keep=0.7)
    d = p.to_device("cuda")
    T, Hq, D = p.q.shape
    ntasks = len(p.seqlens_kv) * Hq * ((p.max_seqlen_q + 127) // 128)
    sched = torch.empty(ntasks, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, bsa.bsa_fp8_schedule_workspace_bytes(len(p.seqlens_kv), Hq, p.max_seqlen_q)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")

    def call(o, l, s):
        bsa.bsa_fp8_schedule(d["cu_seqlens_q"], d["seqlens_kv"], d["block_mask"], num_heads_q=Hq,
                             max_seqlen_q=p.max_seqlen_q, causal=p.causal, workspace=ws, schedule=s)
        bsa.bsa_fp8_prefill_ex(d["q"], d["kcache"], d["vcache"], d["qscale"], d["kscale"], d["vscale"],
                               d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"], d["block_mask"],
                               p.quant_type, p.page_size, max_seqlen_q=p.max_seqlen_q, kv_layout=p.kv_layout,
                               causal=p.causal, softmax_scale=p.softmax_scale, schedule=s, out=o, lse=l)

    say("[gpu] graph schedule + prefill")
    g = capture(lambda: call(out, lse, sched))
    rng = np.random.default_rng(621)
    for r in range(REPLAYS):
        d["block_mask"].copy_(torch.from_numpy(rng.integers(0, 2, size=p.block_mask.shape, dtype=np.uint8)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo = torch.empty_like(out)
        el = torch.empty_like(lse)
        es = torch.empty_like(sched)
        call(eo, el, es)
        torch.cuda.synchronize()
        assert torch.equal(sched, es), f"replay {r}: schedule"
        assert same(out, eo) and same(lse, el), f"replay {r}"
    say("[gpu]   ok")


def test_quantize_append_graph_replays():
    import block_sparse_fp8_amd as bsa
    p = make_problem("tiny", seed=630, lq=(200, 77), lkv=(390, 77), hq=4, hkv=2, quant_type=1, kv_layout=1,
                     page_size=32, keep=0.5)
    a = append_inputs(p, seed=63)
    d = p.to_device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q_in, k_in, v_in = (t(a[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    ks, vs = t(a["kscale"]), t(a["vscale"])
    T, Hq, D = p.q.shape
    q_out = torch.empty((T, Hq, D), dtype=torch.float8_e4m3fn, device="cuda")
    qs_out = torch.empty((T, Hq), dtype=torch.float32, device="cuda")

    def call(kc, vc, ksc, qo, qs):
        bsa.bsa_fp8_quantize_append(q_in, k_in, v_in, d["cu_seqlens_q"], d["seqlens_kv"], d["block_table"],
                                    ks, vs, p.quant_type, p.page_size, kcache=kc, vcache=vc, kscale_cache=ksc,
                                    kv_layout=p.kv_layout, q_out=qo, qscale_out=qs)

    kc, vc, ksc = d["kcache"], d["vcache"], d["kscale"]
    say("[gpu] graph quantize/append")
    g = capture(lambda: call(kc, vc, ksc, q_out, qs_out))
    rng = np.random.default_rng(631)
    for r in range(REPLAYS):
        for x in (q_in, k_in, v_in):
            x.copy_(torch.from_numpy(rng.standard_normal(tuple(x.shape), dtype=np.float32)).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ekc, evc, eksc = kc.clone(), vc.clone(), ksc.clone()
        eqo, eqs = torch.empty_like(q_out), torch.empty_like(qs_out)
        call(ekc, evc, eksc, eqo, eqs)
        torch.cuda.synchronize()
        assert torch.equal(q_out.view(torch.uint8), eqo.view(torch.uint8)) and torch.equal(qs_out, eqs), \
            f"replay {r}: Q"
        assert torch.equal(kc.view(torch.uint8), ekc.view(torch.uint8)), f"replay {r}: K cache"
        assert torch.equal(vc.view(torch.uint8), evc.view(torch.uint8)), f"replay {r}: V cache"
        assert torch.equal(ksc, eksc), f"replay {r}: K descales"
    say("[gpu]   ok")
