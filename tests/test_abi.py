"""The C ABI library: it loads without a GPU, exports every declared symbol, and
rejects bad static arguments with the documented status before any HIP call."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import block_sparse_fp8_amd as bsa
from block_sparse_fp8_amd import Dims, Options

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa_fp8.h")
CONSTRAINTS = json.load(open(os.path.join(ROOT, "tests", "golden", "constraints.json")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.library_path()):
        from block_sparse_fp8_amd import build
        build.build()
    return bsa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_fp8_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "bsa_fp8_prefill" in names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.bsa_fp8_abi_version() == 4


def test_status_strings(lib):
    for s in range(0, 19):
        assert isinstance(bsa.status_string(s), str) and bsa.status_string(s)
    assert bsa.status_string(999) == "unknown status"


def test_status_enum_matches_header():
    text = open(HEADER).read()
    vals = dict((k, int(v)) for k, v in re.findall(r"(BSA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    assert vals["BSA_OK"] == 0
    assert len(set(vals.values())) == len(vals)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def good_dims(**kw):
    d = dict(batch=1, total_q=256, num_heads_q=8, num_heads_kv=2, head_dim=128, num_pages=8,
             max_pages_per_seq=4, max_seqlen_q=256, mask_tiles_q=2, mask_tiles_kv=2, kv_layout=0,
             causal=1, softmax_scale=0.08838834764831845)
    d.update(kw)
    return Dims(**d)


def call(lib, dims, quant=0, page_size=64, mask=FAKE, q=FAKE, out=FAKE, dims_ptr=True):
    return lib.bsa_fp8_prefill(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mask, quant,
                               page_size, ctypes.byref(dims) if dims_ptr else None, out, FAKE, None)


CASES = [
    ("BSA_ERR_HEAD_DIM", dict(head_dim=64), {}),
    ("BSA_ERR_HEAD_DIM", dict(head_dim=256), {}),
    ("BSA_ERR_PAGE_SIZE", {}, dict(page_size=16)),
    ("BSA_ERR_PAGE_SIZE", {}, dict(page_size=128)),
    ("BSA_ERR_GQA", dict(num_heads_q=6, num_heads_kv=4), {}),
    ("BSA_ERR_GQA", dict(num_heads_q=34, num_heads_kv=2), {}),
    ("BSA_ERR_QUANT_TYPE", {}, dict(quant=2)),
    ("BSA_ERR_QUANT_TYPE", {}, dict(quant=-1)),
    ("BSA_ERR_KV_LAYOUT", dict(kv_layout=2), {}),
    ("BSA_ERR_SIZE", dict(batch=-1), {}),
    ("BSA_ERR_SIZE", dict(num_heads_kv=0), {}),
    ("BSA_ERR_SIZE", dict(causal=3), {}),
    ("BSA_ERR_MASK_SHAPE", dict(mask_tiles_q=1), {}),
    ("BSA_ERR_MASK_SHAPE", dict(mask_tiles_kv=0), {}),
    ("BSA_ERR_SOFTMAX_SCALE", dict(softmax_scale=float("nan")), {}),
    ("BSA_ERR_SOFTMAX_SCALE", dict(softmax_scale=float("inf")), {}),
    ("BSA_ERR_SOFTMAX_SCALE", dict(softmax_scale=-0.0883), {}),
    ("BSA_ERR_SOFTMAX_SCALE", dict(softmax_scale=-1e-30), {}),
    ("BSA_ERR_TOO_LARGE", dict(mask_tiles_kv=4097), {}),
    ("BSA_ERR_NULL_POINTER", {}, dict(q=None)),
    ("BSA_ERR_NULL_POINTER", {}, dict(out=None)),
    ("BSA_ERR_NULL_POINTER", {}, dict(dims_ptr=False)),
]


def status_values():
    text = open(HEADER).read()
    return dict((k, int(v)) for k, v in re.findall(r"(BSA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))


@pytest.mark.parametrize("name,dkw,ckw", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_static_validation(lib, name, dkw, ckw):
    assert call(lib, good_dims(**dkw), **ckw) == status_values()[name]


def test_constraints_follow_the_pages(lib):
    """head_dim 128 only, page sizes 32/64, GQA ratio 1..16 (constraint table)."""
    st = status_values()
    for ps in range(1, 129):
        r = call(lib, good_dims(batch=0), page_size=ps)
        assert (r == st["BSA_OK"]) == (ps in CONSTRAINTS["page_sizes"])
    for ratio in range(1, 20):
        r = call(lib, good_dims(batch=0, num_heads_q=ratio, num_heads_kv=1))
        ok = CONSTRAINTS["gqa_ratio_min"] <= ratio <= CONSTRAINTS["gqa_ratio_max"]
        assert (r == st["BSA_OK"]) == ok


def test_empty_grid_returns_ok_without_launch(lib):
    # batch = 0 or max_seqlen_q = 0: nothing to do, no HIP call, null pointers accepted
    z = ctypes.c_void_p(0)
    d = good_dims(batch=0)
    assert lib.bsa_fp8_prefill(z, z, z, z, z, z, z, z, z, z, 0, 64, ctypes.byref(d), z, z, None) == 0
    d = good_dims(max_seqlen_q=0, total_q=0)
    assert lib.bsa_fp8_prefill(z, z, z, z, z, z, z, z, z, z, 0, 64, ctypes.byref(d), z, z, None) == 0


def test_failed_call_leaves_outputs_untouched(lib):
    out = np.full(64, 7, dtype=np.uint16)
    r = call(lib, good_dims(head_dim=64), out=ctypes.c_void_p(out.ctypes.data))
    assert r == status_values()["BSA_ERR_HEAD_DIM"]
    assert np.all(out == 7)


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(4, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        bsa.bsa_fp8_prefill(x, x, x, x, x, x, x, x, x, None, 0, 64, max_seqlen_q=4)


def call_ex(lib, dims, opts=None, quant=0, page_size=64, mask=FAKE, q=FAKE, out=FAKE):
    return lib.bsa_fp8_prefill_ex(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mask, quant,
                                  page_size, ctypes.byref(dims),
                                  None if opts is None else ctypes.byref(opts), out, FAKE, None)


def opts(**kw):
    return Options(**kw)


EX_CASES = [
    ("BSA_ERR_Q_LAYOUT", dict(q_layout=2), {}),
    ("BSA_ERR_Q_LAYOUT", dict(q_layout=-1), {}),
    ("BSA_ERR_P_SCALE", dict(p_scale=-1.0), {}),
    ("BSA_ERR_P_SCALE", dict(p_scale=448.5), {}),
    ("BSA_ERR_P_SCALE", dict(p_scale=float("nan")), {}),
    ("BSA_ERR_P_SCALE", dict(p_scale=float("inf")), {}),
    ("BSA_ERR_SPARSE_FORM", dict(sparse_indices=0x1000, sparse_seq_len=0x1000), {}),   # + mask
    ("BSA_ERR_SPARSE_FORM", dict(sparse_indices=0x1000), dict(mask=None)),
    ("BSA_ERR_SPARSE_FORM", dict(sparse_seq_len=0x1000), dict(mask=None)),
    ("BSA_ERR_SCHEDULE", dict(schedule=0x1000, schedule_len=3), {}),
    ("BSA_ERR_MASK_SHAPE", dict(sparse_indices=0x1000, sparse_seq_len=0x1000),
     dict(mask=None, dims=dict(mask_tiles_q=1))),
    ("BSA_ERR_TOO_LARGE", dict(sparse_indices=0x1000, sparse_seq_len=0x1000),
     dict(mask=None, dims=dict(mask_tiles_kv=4097))),
    ("BSA_ERR_HEAD_DIM", {}, dict(dims=dict(head_dim=64))),
    ("BSA_ERR_PAGE_SIZE", {}, dict(page_size=48)),
    ("BSA_ERR_QUANT_TYPE", {}, dict(quant=3)),
]


@pytest.mark.parametrize("name,okw,ckw", EX_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(EX_CASES)])
def test_ex_static_validation(lib, name, okw, ckw):
    ckw = dict(ckw)
    d = good_dims(**ckw.pop("dims", {}))
    assert call_ex(lib, d, opts(**okw), **ckw) == status_values()[name]


def test_ex_accepts_valid_options_without_launch(lib):
    # batch = 0: every static check runs, nothing is launched.
    st = status_values()
    d = good_dims(batch=0)
    for ps in (0.0, 1e-3, 1.0, 256.0, 300.0, 448.0):
        assert call_ex(lib, d, opts(p_scale=ps)) == st["BSA_OK"], ps
    assert call_ex(lib, d, opts(q_layout=1)) == st["BSA_OK"]
    assert call_ex(lib, d, None) == st["BSA_OK"]
    assert call_ex(lib, d, opts(sparse_indices=0x1000, sparse_seq_len=0x1000), mask=None) == st["BSA_OK"]
    # the task count is B * Hq * ceil(max_seqlen_q / 128) = 0 here
    assert call_ex(lib, d, opts(schedule=0x1000, schedule_len=0)) == st["BSA_OK"]
    assert call_ex(lib, d, opts(schedule=0x1000, schedule_len=1)) == st["BSA_ERR_SCHEDULE"]


def test_schedule_workspace_bytes(lib):
    d = good_dims()                   # 1 * 8 * 2 = 16 tasks
    n = lib.bsa_fp8_schedule_workspace_bytes(ctypes.byref(d))
    assert n >= 16 * 4 * 2 + 1024 * 4 and n % 4 == 0
    d = good_dims(batch=9, num_heads_q=16, num_heads_kv=16, max_seqlen_q=128 * 100)   # 14400 tasks
    n = lib.bsa_fp8_schedule_workspace_bytes(ctypes.byref(d))
    assert n >= 14400 * 8 + 15 * 1024 * 4
    assert lib.bsa_fp8_schedule_workspace_bytes(ctypes.byref(good_dims(batch=0))) == 0
    assert lib.bsa_fp8_schedule_workspace_bytes(ctypes.byref(good_dims(head_dim=64))) == -1
    assert lib.bsa_fp8_schedule_workspace_bytes(None) == -1


def test_schedule_static_validation(lib):
    st = status_values()
    d = good_dims()
    z = ctypes.c_void_p(0)
    sched = lambda dims, mask=FAKE, o=None, ws=FAKE, out=FAKE, cu=FAKE: lib.bsa_fp8_schedule(
        cu, FAKE, mask, ctypes.byref(dims), None if o is None else ctypes.byref(o), ws, out, None)
    assert sched(d, ws=z) == st["BSA_ERR_NULL_POINTER"]
    assert sched(d, out=z) == st["BSA_ERR_NULL_POINTER"]
    assert sched(d, cu=z) == st["BSA_ERR_NULL_POINTER"]
    assert sched(d, o=opts(sparse_indices=0x1000, sparse_seq_len=0x1000)) == st["BSA_ERR_SPARSE_FORM"]
    assert sched(good_dims(mask_tiles_q=1)) == st["BSA_ERR_MASK_SHAPE"]
    assert sched(good_dims(head_dim=64)) == st["BSA_ERR_HEAD_DIM"]
    # only the sparsity fields of the options are read: a bad layout is ignored
    assert sched(good_dims(batch=0), o=opts(q_layout=7, p_scale=-1.0)) == st["BSA_OK"]
    assert sched(good_dims(batch=0), ws=z, out=z, cu=z) == st["BSA_OK"]


def quant_call(lib, dims, q_in=FAKE, k_in=FAKE, v_in=FAKE, kscale=FAKE, kscale_cache=FAKE,
               q_out=FAKE, qscale_out=FAKE, quant=0, page_size=64, mode=0):
    return lib.bsa_fp8_quantize_append(q_in, k_in, v_in, FAKE, FAKE, FAKE, kscale, FAKE, quant,
                                       page_size, mode, ctypes.byref(dims), q_out, qscale_out,
                                       FAKE, FAKE, kscale_cache, None)


def test_quantize_append_static_validation(lib):
    st = status_values()
    d = good_dims()
    z = None
    assert quant_call(lib, d, mode=2) == st["BSA_ERR_SCALE_MODE"]
    assert quant_call(lib, d, mode=-1) == st["BSA_ERR_SCALE_MODE"]
    assert quant_call(lib, d, v_in=z) == st["BSA_ERR_NULL_POINTER"]          # K without V
    assert quant_call(lib, d, k_in=z) == st["BSA_ERR_NULL_POINTER"]          # V without K
    assert quant_call(lib, d, kscale=z, quant=0) == st["BSA_ERR_NULL_POINTER"]
    assert quant_call(lib, d, kscale_cache=z, quant=1) == st["BSA_ERR_NULL_POINTER"]
    assert quant_call(lib, d, q_out=z) == st["BSA_ERR_NULL_POINTER"]
    assert quant_call(lib, d, qscale_out=z) == st["BSA_ERR_NULL_POINTER"]
    assert quant_call(lib, d, page_size=48) == st["BSA_ERR_PAGE_SIZE"]
    assert quant_call(lib, d, quant=5) == st["BSA_ERR_QUANT_TYPE"]
    assert quant_call(lib, good_dims(head_dim=64)) == st["BSA_ERR_HEAD_DIM"]
    assert quant_call(lib, good_dims(num_heads_q=6, num_heads_kv=4)) == st["BSA_ERR_GQA"]
    assert quant_call(lib, good_dims(batch=0)) == st["BSA_ERR_SIZE"]         # K/V rows need a sequence
    # nothing to do: no launch, OK
    assert quant_call(lib, d, q_in=z, k_in=z, v_in=z, q_out=z, qscale_out=z) == st["BSA_OK"]
    assert quant_call(lib, good_dims(total_q=0)) == st["BSA_OK"]
    # the parts that are skipped need no pointers
    assert quant_call(lib, good_dims(total_q=0), k_in=z, v_in=z, kscale=z, kscale_cache=z) == st["BSA_OK"]


def test_sparse_decode_static_validation(lib):
    from block_sparse_fp8_amd import DecodeDims
    st = status_values()

    def dd(**kw):
        d = dict(batch=2, s_q=2, num_heads_q=128, topk=64, num_pages=10, page_size=64,
                 softmax_scale=0.0417)
        d.update(kw)
        return DecodeDims(**d)

    def call_dec(dims, q=FAKE, out=FAKE, dims_ptr=True):
        return lib.bsa_fp8_sparse_decode(q, FAKE, FAKE, ctypes.byref(dims) if dims_ptr else None, out,
                                         FAKE, None)

    assert call_dec(dd(), dims_ptr=False) == st["BSA_ERR_NULL_POINTER"]
    assert call_dec(dd(num_heads_q=96)) == st["BSA_ERR_GQA"]
    assert call_dec(dd(num_heads_q=0)) == st["BSA_ERR_SIZE"]
    assert call_dec(dd(topk=0)) == st["BSA_ERR_SIZE"]
    assert call_dec(dd(batch=-1)) == st["BSA_ERR_SIZE"]
    assert call_dec(dd(page_size=0)) == st["BSA_ERR_PAGE_SIZE"]
    assert call_dec(dd(page_size=-64)) == st["BSA_ERR_PAGE_SIZE"]
    assert call_dec(dd(softmax_scale=float("nan"))) == st["BSA_ERR_SOFTMAX_SCALE"]
    assert call_dec(dd(num_pages=2 ** 30, page_size=64)) == st["BSA_ERR_TOO_LARGE"]
    assert call_dec(dd(), q=None) == st["BSA_ERR_NULL_POINTER"]
    assert call_dec(dd(), out=None) == st["BSA_ERR_NULL_POINTER"]
    z = ctypes.c_void_p(0)
    assert lib.bsa_fp8_sparse_decode(z, z, z, ctypes.byref(dd(batch=0)), z, z, None) == st["BSA_OK"]
    assert lib.bsa_fp8_sparse_decode(z, z, z, ctypes.byref(dd(s_q=0)), z, z, None) == st["BSA_OK"]


def test_split_decode_static_validation(lib):
    from block_sparse_fp8_amd import DecodeDims
    st = status_values()

    def dd(**kw):
        d = dict(batch=2, s_q=2, num_heads_q=128, topk=64, num_pages=10, page_size=64,
                 softmax_scale=0.0417)
        d.update(kw)
        return DecodeDims(**d)

    def call_ex(dims, splits, ws=FAKE):
        return lib.bsa_fp8_sparse_decode_ex(FAKE, FAKE, FAKE, ctypes.byref(dims), splits, ws, FAKE, FAKE,
                                            None)

    assert call_ex(dd(), 0) == st["BSA_ERR_SIZE"]
    assert call_ex(dd(), 257) == st["BSA_ERR_SIZE"]
    assert call_ex(dd(), 2, ws=None) == st["BSA_ERR_NULL_POINTER"]
    assert call_ex(dd(), 2, ws=ctypes.c_void_p(0x1008)) == st["BSA_ERR_SIZE"]   # not 16-byte aligned
    # one workgroup holds at most 8192 entries: a list of 16384 needs two parts
    assert call_ex(dd(topk=16384), 1) == st["BSA_ERR_TOO_LARGE"]
    assert lib.bsa_fp8_sparse_decode(FAKE, FAKE, FAKE, ctypes.byref(dd(topk=16384)), FAKE, FAKE,
                                     None) == st["BSA_ERR_TOO_LARGE"]
    # 8193 entries are 257 blocks: two parts of 129 blocks (4128 entries) fit
    assert call_ex(dd(topk=8193, batch=0), 2) == st["BSA_OK"]
    assert call_ex(dd(topk=8193), 1) == st["BSA_ERR_TOO_LARGE"]
    assert call_ex(dd(topk=2 ** 21 + 1), 256) == st["BSA_ERR_TOO_LARGE"]
    z = ctypes.c_void_p(0)
    assert lib.bsa_fp8_sparse_decode_ex(z, z, z, ctypes.byref(dd(batch=0)), 4, z, z, z, None) == st["BSA_OK"]


def test_noalloc_decode_static_validation(lib):
    """The no-allocation decode rejects, before any HIP call, partial results
    beyond its static scratch, and otherwise validates like the split decode."""
    from block_sparse_fp8_amd import DecodeDims
    st = status_values()
    d = DecodeDims(batch=64, s_q=2, num_heads_q=128, topk=2048, num_pages=10, page_size=64,
                   softmax_scale=0.0417)
    call = lambda dims, n: lib.bsa_fp8_sparse_decode_noalloc(FAKE, FAKE, FAKE, ctypes.byref(dims), n,  # noqa: E731
                                                             FAKE, FAKE, None)
    per_part = 64 * 2 * 128 * 513 * 4                 # 33.6 MB: two parts exceed 64 MiB
    assert per_part * 2 > 64 * 1024 * 1024
    assert call(d, 2) == st["BSA_ERR_SCRATCH"]
    assert call(d, 257) == st["BSA_ERR_SIZE"]
    assert call(DecodeDims(batch=64, s_q=2, num_heads_q=96, topk=2048, num_pages=10, page_size=64,
                           softmax_scale=0.0417), 2) == st["BSA_ERR_GQA"]
    assert lib.bsa_fp8_sparse_decode_noalloc(FAKE, FAKE, FAKE, None, 2, FAKE, FAKE, None) == \
        st["BSA_ERR_NULL_POINTER"]
    z = ctypes.c_void_p(0)
    # nothing to do: no launch and no scratch lookup
    assert lib.bsa_fp8_sparse_decode_noalloc(z, z, z, ctypes.byref(DecodeDims(
        batch=0, s_q=2, num_heads_q=128, topk=64, num_pages=10, page_size=64, softmax_scale=0.04)), 4, z, z,
        None) == st["BSA_OK"]


def test_split_decode_sizes(lib):
    from block_sparse_fp8_amd import DecodeDims

    def dd(**kw):
        d = dict(batch=2, s_q=2, num_heads_q=128, topk=2048, num_pages=10, page_size=64,
                 softmax_scale=0.0417)
        d.update(kw)
        return DecodeDims(**d)

    ws = lambda d, n: lib.bsa_fp8_sparse_decode_workspace_bytes(ctypes.byref(d), n)  # noqa: E731
    assert ws(dd(), 1) == 0
    assert ws(dd(), 3) == 3 * 2 * 2 * 128 * 513 * 4
    assert ws(dd(), 0) == -1 and ws(dd(), 257) == -1 and ws(dd(batch=-1), 2) == -1
    assert lib.bsa_fp8_sparse_decode_workspace_bytes(None, 2) == -1
    assert bsa.bsa_fp8_sparse_decode_workspace_bytes(1, 2, 64, 5) == 5 * 2 * 64 * 513 * 4
    ns = lambda **kw: lib.bsa_fp8_sparse_decode_num_splits(ctypes.byref(dd(**kw)))  # noqa: E731
    # 128 heads are one workgroup per query token; B*s_q = 4 -> 64 parts wanted,
    # but 2048 entries are 64 blocks, at least 2 per part -> 32
    assert ns() == 32
    assert ns(batch=8) == 16                         # 16 query tokens x 16 parts = 256 workgroups
    assert ns(batch=128) == 1                        # 256 workgroups already
    assert ns(batch=1, s_q=1, topk=65536) == 256     # 2048 blocks: 256 parts of 8
    assert ns(batch=128, topk=65536) == 8            # the list must fit: 8 parts of 8192
    assert ns(batch=1, s_q=1, num_heads_q=64, topk=128) == 2   # 4 blocks: 2 parts of 2
    assert ns(batch=1, s_q=1, num_heads_q=64, topk=32) == 1    # one block cannot be split
    assert ns(num_heads_q=96) == 1 and ns(topk=0) == 1
    assert lib.bsa_fp8_sparse_decode_num_splits(None) == 1
    for kw in (dict(), dict(batch=1, s_q=1, topk=100000), dict(batch=64, topk=30000)):
        d = dd(**kw)
        n = lib.bsa_fp8_sparse_decode_num_splits(ctypes.byref(d))
        blocks = -(-d.topk // 32)
        assert 1 <= n <= 256 and -(-blocks // n) * 32 <= 8192
