"""Block-sparse FP8 (E4M3) attention prefill over a paged KV cache, MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/bsa_fp8.h``: it
checks tensor devices/dtypes, allocates outputs with torch, passes raw device
pointers and torch's current stream, and raises on a non-zero status.  Every
step of the computation runs in the HIP library ``libbsa_fp8.so``; there is no
other code path.  If the library has not been built, importing this package
still works but every call raises ``RuntimeError``.
"""
import ctypes
import enum
import math
import os

import torch

__all__ = [
    "QuantType",
    "KVLayout",
    "BsaError",
    "QLayout",
    "QKPrecision",
    "bsa_fp8_prefill",
    "bsa_fp8_prefill_ex",
    "bsa_fp8_schedule",
    "bsa_fp8_schedule_workspace_bytes",
    "bsa_fp8_quantize_append",
    "bsa_fp8_sparse_decode",
    "bsa_fp8_sparse_decode_ex",
    "bsa_fp8_sparse_decode_noalloc",
    "bsa_fp8_sparse_decode_workspace_bytes",
    "bsa_fp8_sparse_decode_num_splits",
    "DecodeDims",
    "ScaleMode",
    "attention_with_kvcache_blocksparse_prefill_fp8",
    "library_path",
    "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libbsa_fp8.so"


def library_path():
    return os.path.join(_HERE, LIB_NAME)


class QuantType(enum.IntEnum):
    """Quantisation schemes (hpc-ops article, "FP8 Tensor Core compute")."""
    QPERTOKEN_PERHEAD_KPERTENSOR_VPERTENSOR = 0
    QPERTOKEN_PERHEAD_KPERTOKEN_PERHEAD_VPERHEAD = 1


class KVLayout(enum.IntEnum):
    NHD = 0  # [num_pages, page_size, Hkv, 128]
    HND = 1  # [num_pages, Hkv, page_size, 128]


class QLayout(enum.IntEnum):
    """Query layouts ("Quant Block Sparse Attention", "Key parameters")."""
    TND = 0  # q [T, Hq, 128], qscale [T, Hq]
    NTD = 1  # q [Hq, T, 128], qscale [Hq, T]


class QKPrecision(enum.IntEnum):
    """Matrix path of the prefill's Q.K^T products (bsa_qk_precision)."""
    DEFAULT = 0  # the library's choice
    F16 = 1      # E4M3 widened exactly to f16, f16 matrix products
    FP8 = 2      # E4M3 operands, one FP8 matrix product per K operand
    FP8_SPLIT = 3  # E4M3 operands, two FP8 products per K operand (magnitude-split Q)


class ScaleMode(enum.IntEnum):
    """Descale rule of the quantisation step (FlashMLA FP8 KV-cache article)."""
    AMAX = 0       # amax / 448
    AMAX_POW2 = 1  # amax / 448 rounded up to a power of two


class BsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"bsa_fp8_prefill failed (status {status}): {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("mask_tiles_q", ctypes.c_int32),
        ("mask_tiles_kv", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


_lib_handle = None


class Options(ctypes.Structure):
    _fields_ = [
        ("q_layout", ctypes.c_int32),
        ("p_scale", ctypes.c_float),
        ("sparse_indices", ctypes.c_void_p),
        ("sparse_seq_len", ctypes.c_void_p),
        ("schedule", ctypes.c_void_p),
        ("schedule_len", ctypes.c_int32),
        ("qk_precision", ctypes.c_int32),
    ]


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


def load_library():
    """Load libbsa_fp8.so (once).  Raises RuntimeError if it is not built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m block_sparse_fp8_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.bsa_fp8_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_int, ctypes.c_int, ctypes.POINTER(Dims), vp, vp, vp]
    lib.bsa_fp8_prefill.restype = ctypes.c_int
    lib.bsa_fp8_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_int, ctypes.c_int, ctypes.POINTER(Dims),
                                       ctypes.POINTER(Options), vp, vp, vp]
    lib.bsa_fp8_prefill_ex.restype = ctypes.c_int
    lib.bsa_fp8_schedule_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    lib.bsa_fp8_schedule_workspace_bytes.restype = ctypes.c_longlong
    lib.bsa_fp8_schedule.argtypes = [vp, vp, vp, ctypes.POINTER(Dims), ctypes.POINTER(Options),
                                     vp, vp, vp]
    lib.bsa_fp8_schedule.restype = ctypes.c_int
    lib.bsa_fp8_quantize_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.POINTER(Dims),
                                            vp, vp, vp, vp, vp, vp]
    lib.bsa_fp8_quantize_append.restype = ctypes.c_int
    lib.bsa_fp8_sparse_decode.argtypes = [vp, vp, vp, ctypes.POINTER(DecodeDims), vp, vp, vp]
    lib.bsa_fp8_sparse_decode.restype = ctypes.c_int
    lib.bsa_fp8_sparse_decode_ex.argtypes = [vp, vp, vp, ctypes.POINTER(DecodeDims),
                                             ctypes.c_int, vp, vp, vp, vp]
    lib.bsa_fp8_sparse_decode_ex.restype = ctypes.c_int
    lib.bsa_fp8_sparse_decode_noalloc.argtypes = [vp, vp, vp, ctypes.POINTER(DecodeDims), ctypes.c_int,
                                                  vp, vp, vp]
    lib.bsa_fp8_sparse_decode_noalloc.restype = ctypes.c_int
    lib.bsa_fp8_sparse_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeDims), ctypes.c_int]
    lib.bsa_fp8_sparse_decode_workspace_bytes.restype = ctypes.c_longlong
    lib.bsa_fp8_sparse_decode_num_splits.argtypes = [ctypes.POINTER(DecodeDims)]
    lib.bsa_fp8_sparse_decode_num_splits.restype = ctypes.c_int
    lib.bsa_fp8_status_string.argtypes = [ctypes.c_int]
    lib.bsa_fp8_status_string.restype = ctypes.c_char_p
    lib.bsa_fp8_abi_version.argtypes = []
    lib.bsa_fp8_abi_version.restype = ctypes.c_int
    _lib_handle = lib
    return lib


def status_string(status):
    return load_library().bsa_fp8_status_string(int(status)).decode()


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtypes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _sparsity_shape(block_mask, sparse_indices, sparse_seq_len, device):
    """(mask_tiles_q, mask_tiles_kv) of the sparsity argument, after checks."""
    if block_mask is not None:
        _check("block_mask", block_mask, (torch.uint8, torch.bool), device)
        if block_mask.dim() != 4:
            raise ValueError("block_mask must be [B, Hq, mask_tiles_q, mask_tiles_kv]")
        return block_mask.shape[2], block_mask.shape[3]
    if sparse_indices is not None or sparse_seq_len is not None:
        if sparse_indices is None or sparse_seq_len is None:
            raise ValueError("sparse_indices and sparse_seq_len come together")
        _check("sparse_indices", sparse_indices, (torch.int32,), device)
        _check("sparse_seq_len", sparse_seq_len, (torch.int32,), device)
        if sparse_indices.dim() != 4 or sparse_seq_len.shape != sparse_indices.shape[:3]:
            raise ValueError("sparse_indices must be [B, Hq, Qb, Kb] and sparse_seq_len [B, Hq, Qb]")
        return sparse_indices.shape[2], sparse_indices.shape[3]
    return 0, 0


def _options(q_layout, p_scale, sparse_indices, sparse_seq_len, schedule, qk_precision=0):
    return Options(q_layout=int(q_layout), p_scale=0.0 if p_scale is None else float(p_scale),
                   sparse_indices=None if sparse_indices is None else sparse_indices.data_ptr(),
                   sparse_seq_len=None if sparse_seq_len is None else sparse_seq_len.data_ptr(),
                   schedule=None if schedule is None else schedule.data_ptr(),
                   schedule_len=0 if schedule is None else schedule.numel(),
                   qk_precision=int(qk_precision))


def _prefill(entry, q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
             seqlens_kv, block_mask, quant_type, page_size, max_seqlen_q, kv_layout, causal,
             softmax_scale, out, lse, return_lse, stream, q_layout=QLayout.TND, p_scale=None,
             sparse_indices=None, sparse_seq_len=None, schedule=None, qk_precision=0):
    device = q.device
    if device.type != "cuda":
        raise ValueError(entry + " runs on a GPU; q is on " + str(device))
    _check("q", q, _FP8, device)
    _check("kcache", kcache, _FP8, device)
    _check("vcache", vcache, _FP8, device)
    for name, t in (("qscale", qscale), ("kscale", kscale), ("vscale", vscale)):
        _check(name, t, (torch.float32,), device)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("block_table", block_table),
                    ("seqlens_kv", seqlens_kv)):
        _check(name, t, (torch.int32,), device)
    mt, mkv = _sparsity_shape(block_mask, sparse_indices, sparse_seq_len, device)
    if schedule is not None:
        _check("schedule", schedule, (torch.int32,), device)
    if q.dim() != 3 or kcache.dim() != 4 or vcache.shape != kcache.shape:
        raise ValueError("q must be 3-D; kcache/vcache must be 4-D and of equal shape")
    q_layout = QLayout(int(q_layout))
    if q_layout == QLayout.TND:
        T, Hq, D = q.shape
    else:
        Hq, T, D = q.shape
    kv_layout = KVLayout(int(kv_layout))
    Hkv = kcache.shape[2] if kv_layout == KVLayout.NHD else kcache.shape[1]
    B = seqlens_kv.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=device)
    else:
        _check("out", out, (torch.bfloat16,), device)
    if lse is None and return_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=device)
    elif lse is not None:
        _check("lse", lse, (torch.float32,), device)
    dims = Dims(batch=B, total_q=T, num_heads_q=Hq, num_heads_kv=Hkv, head_dim=D,
                num_pages=kcache.shape[0], max_pages_per_seq=block_table.shape[1],
                max_seqlen_q=int(max_seqlen_q), mask_tiles_q=mt, mask_tiles_kv=mkv,
                kv_layout=int(kv_layout), causal=1 if causal else 0,
                softmax_scale=float(softmax_scale))
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    lib = load_library()
    mask_u8 = block_mask.view(torch.uint8) if block_mask is not None else None
    args = [_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(qscale), _ptr(kscale), _ptr(vscale),
            _ptr(cu_seqlens_q), _ptr(block_table), _ptr(seqlens_kv), _ptr(mask_u8),
            int(quant_type), int(page_size), ctypes.byref(dims)]
    if entry == "bsa_fp8_prefill_ex":
        opts = _options(q_layout, p_scale, sparse_indices, sparse_seq_len, schedule, qk_precision)
        args.append(ctypes.byref(opts))
    args += [_ptr(out), _ptr(lse), ctypes.c_void_p(stream)]
    status = getattr(lib, entry)(*args)
    if status != 0:
        raise BsaError(status, status_string(status))
    return out, lse


def bsa_fp8_prefill(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
                    seqlens_kv, block_mask, quant_type, page_size, *, max_seqlen_q,
                    kv_layout=KVLayout.NHD, causal=True, softmax_scale=None,
                    out=None, lse=None, return_lse=True, stream=None):
    """Call the C entry point of the same name.  Returns (out, lse).

    Shapes and meaning are those of ``include/bsa_fp8.h``.  ``out`` (bf16
    [T,Hq,128]) and ``lse`` (float32 [Hq,T]) are allocated when not given.
    """
    return _prefill("bsa_fp8_prefill", q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q,
                    block_table, seqlens_kv, block_mask, quant_type, page_size, max_seqlen_q,
                    kv_layout, causal, softmax_scale, out, lse, return_lse, stream)


def bsa_fp8_prefill_ex(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
                       seqlens_kv, block_mask, quant_type, page_size, *, max_seqlen_q,
                       kv_layout=KVLayout.NHD, causal=True, softmax_scale=None,
                       q_layout=QLayout.TND, p_scale=None, sparse_indices=None,
                       sparse_seq_len=None, schedule=None, qk_precision=QKPrecision.DEFAULT,
                       out=None, lse=None, return_lse=True, stream=None):
    """Call the C entry point of the same name: bsa_fp8_prefill plus the query
    layout (q [Hq,T,128] and qscale [Hq,T] for NTD), the P-scale (None = 256),
    the index-list sparsity (sparse_indices int32 [B,Hq,Qb,Kb] with
    sparse_seq_len int32 [B,Hq,Qb], instead of block_mask), a task order
    from ``bsa_fp8_schedule`` and the matrix path of Q.K^T (QKPrecision).
    Returns (out, lse); out is TND."""
    return _prefill("bsa_fp8_prefill_ex", q, kcache, vcache, qscale, kscale, vscale,
                    cu_seqlens_q, block_table, seqlens_kv, block_mask, quant_type, page_size,
                    max_seqlen_q, kv_layout, causal, softmax_scale, out, lse, return_lse, stream,
                    q_layout=q_layout, p_scale=p_scale, sparse_indices=sparse_indices,
                    sparse_seq_len=sparse_seq_len, schedule=schedule, qk_precision=qk_precision)


def _schedule_dims(batch, num_heads_q, max_seqlen_q, mt, mkv, causal):
    # The pre-pass reads only the sequence lengths and the sparsity; the other
    # fields take any valid value.
    return Dims(batch=batch, total_q=0, num_heads_q=num_heads_q, num_heads_kv=num_heads_q,
                head_dim=128, num_pages=0, max_pages_per_seq=0, max_seqlen_q=int(max_seqlen_q),
                mask_tiles_q=mt, mask_tiles_kv=mkv, kv_layout=0, causal=1 if causal else 0,
                softmax_scale=1.0)


def bsa_fp8_schedule_workspace_bytes(batch, num_heads_q, max_seqlen_q):
    """Device workspace (bytes) the scheduling pre-pass needs."""
    dims = _schedule_dims(batch, num_heads_q, max_seqlen_q, 1, 1, True)
    n = load_library().bsa_fp8_schedule_workspace_bytes(ctypes.byref(dims))
    if n < 0:
        raise ValueError("invalid sizes for the scheduling pre-pass")
    return n


def bsa_fp8_schedule(cu_seqlens_q, seqlens_kv, block_mask=None, *, num_heads_q, max_seqlen_q,
                     causal=True, sparse_indices=None, sparse_seq_len=None, workspace=None,
                     schedule=None, stream=None):
    """Call the C entry point of the same name: the task order (int32
    [B*Hq*ceil(max_seqlen_q/128)], decreasing cost, then increasing task id) for
    ``bsa_fp8_prefill_ex``.  The workspace is allocated when not given."""
    device = seqlens_kv.device
    if device.type != "cuda":
        raise ValueError("bsa_fp8_schedule runs on a GPU; seqlens_kv is on " + str(device))
    _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), device)
    _check("seqlens_kv", seqlens_kv, (torch.int32,), device)
    mt, mkv = _sparsity_shape(block_mask, sparse_indices, sparse_seq_len, device)
    B = seqlens_kv.shape[0]
    dims = _schedule_dims(B, num_heads_q, max_seqlen_q, mt, mkv, causal)
    lib = load_library()
    nbytes = lib.bsa_fp8_schedule_workspace_bytes(ctypes.byref(dims))
    if nbytes < 0:
        raise ValueError("invalid sizes for the scheduling pre-pass")
    ntasks = B * num_heads_q * ((int(max_seqlen_q) + 127) // 128)
    if schedule is None:
        schedule = torch.empty(ntasks, dtype=torch.int32, device=device)
    else:
        _check("schedule", schedule, (torch.int32,), device)
        if schedule.numel() != ntasks:
            raise ValueError(f"schedule must hold {ntasks} task ids")
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must hold {nbytes} bytes")
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    mask_u8 = block_mask.view(torch.uint8) if block_mask is not None else None
    opts = _options(QLayout.TND, None, sparse_indices, sparse_seq_len, None)
    status = lib.bsa_fp8_schedule(_ptr(cu_seqlens_q), _ptr(seqlens_kv), _ptr(mask_u8),
                                  ctypes.byref(dims), ctypes.byref(opts), _ptr(workspace),
                                  _ptr(schedule), ctypes.c_void_p(stream))
    if status != 0:
        raise BsaError(status, status_string(status))
    return schedule


def bsa_fp8_quantize_append(q_in, k_in, v_in, cu_seqlens_q, seqlens_kv, block_table, kscale,
                            vscale, quant_type, page_size, *, kcache, vcache, kscale_cache=None,
                            kv_layout=KVLayout.NHD, scale_mode=ScaleMode.AMAX, q_out=None,
                            qscale_out=None, stream=None):
    """Call the C entry point of the same name: quantise the bfloat16 query
    chunk (q_in [T,Hq,128]) to E4M3 with per-(token, head) descales, and append
    the chunk's keys and values (k_in, v_in [T,Hkv,128]) to the paged caches in
    place (per-token K descales into kscale_cache for quant type 1).  q_in or
    k_in/v_in may be None to skip that part.  Returns (q_out, qscale_out)."""
    ref = q_in if q_in is not None else k_in
    if ref is None:
        raise ValueError("nothing to do: q_in and k_in are both None")
    device = ref.device
    if device.type != "cuda":
        raise ValueError("bsa_fp8_quantize_append runs on a GPU; input is on " + str(device))
    for name, t in (("q_in", q_in), ("k_in", k_in), ("v_in", v_in)):
        if t is not None:
            _check(name, t, (torch.bfloat16,), device)
            if t.dim() != 3 or t.shape[2] != 128:
                raise ValueError(f"{name} must be [T, heads, 128]")
    kv_layout = KVLayout(int(kv_layout))
    T = ref.shape[0]
    Hq = q_in.shape[1] if q_in is not None else 1
    Hkv = Hq   # without K/V the kv-head count only needs to be a valid GQA ratio
    if k_in is not None:
        if v_in is None or v_in.shape != k_in.shape:
            raise ValueError("k_in and v_in come together, with equal shapes")
        for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqlens_kv", seqlens_kv),
                        ("block_table", block_table)):
            _check(name, t, (torch.int32,), device)
        _check("kcache", kcache, _FP8, device)
        _check("vcache", vcache, _FP8, device)
        _check("vscale", vscale, (torch.float32,), device)
        if kscale is not None:
            _check("kscale", kscale, (torch.float32,), device)
        if kscale_cache is not None:
            _check("kscale_cache", kscale_cache, (torch.float32,), device)
        Hkv = k_in.shape[1]
        if q_in is not None and Hq % Hkv != 0:
            raise ValueError("num_heads_q must be a multiple of num_heads_kv")
    if q_in is None:
        Hq = Hkv
    B = seqlens_kv.shape[0] if seqlens_kv is not None else 0
    if q_in is not None:
        if q_out is None:
            q_out = torch.empty(q_in.shape, dtype=torch.float8_e4m3fn, device=device)
        else:
            _check("q_out", q_out, _FP8, device)
        if qscale_out is None:
            qscale_out = torch.empty(q_in.shape[:2], dtype=torch.float32, device=device)
        else:
            _check("qscale_out", qscale_out, (torch.float32,), device)
    dims = Dims(batch=B, total_q=T, num_heads_q=Hq, num_heads_kv=Hkv, head_dim=128,
                num_pages=kcache.shape[0] if kcache is not None else 0,
                max_pages_per_seq=block_table.shape[1] if block_table is not None else 0,
                max_seqlen_q=0, mask_tiles_q=0, mask_tiles_kv=0, kv_layout=int(kv_layout),
                causal=1, softmax_scale=1.0)
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    status = load_library().bsa_fp8_quantize_append(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(cu_seqlens_q), _ptr(seqlens_kv),
        _ptr(block_table), _ptr(kscale), _ptr(vscale), int(quant_type), int(page_size),
        int(scale_mode), ctypes.byref(dims), _ptr(q_out), _ptr(qscale_out), _ptr(kcache),
        _ptr(vcache), _ptr(kscale_cache), ctypes.c_void_p(stream))
    if status != 0:
        raise BsaError(status, status_string(status))
    return q_out, qscale_out


def _decode_dims(batch, s_q, num_heads_q, topk, num_pages=0, page_size=64, softmax_scale=1.0):
    return DecodeDims(batch=batch, s_q=s_q, num_heads_q=num_heads_q, topk=topk, num_pages=num_pages,
                      page_size=page_size, softmax_scale=float(softmax_scale))


def bsa_fp8_sparse_decode_workspace_bytes(batch, s_q, num_heads_q, num_splits):
    """Call the C entry point of the same name: bytes of the split-list
    decode's workspace (0 for one part)."""
    dims = _decode_dims(batch, s_q, num_heads_q, 1)
    n = load_library().bsa_fp8_sparse_decode_workspace_bytes(ctypes.byref(dims), int(num_splits))
    if n < 0:
        raise ValueError("invalid sizes or num_splits for the decode workspace")
    return n


def bsa_fp8_sparse_decode_num_splits(batch, s_q, num_heads_q, topk):
    """Call the C entry point of the same name: a part count that fills the
    chip and keeps each part's list within one workgroup."""
    return load_library().bsa_fp8_sparse_decode_num_splits(
        ctypes.byref(_decode_dims(batch, s_q, num_heads_q, topk)))


def _sparse_decode(q, kv_cache, indices, softmax_scale, out, lse, return_lse, stream, num_splits,
                   workspace):
    device = q.device
    if device.type != "cuda":
        raise ValueError("bsa_fp8_sparse_decode runs on a GPU; q is on " + str(device))
    _check("q", q, (torch.bfloat16,), device)
    _check("kv_cache", kv_cache, (torch.uint8,), device)
    _check("indices", indices, (torch.int32,), device)
    if q.dim() != 4 or q.shape[3] != 576:
        raise ValueError("q must be [B, s_q, h_q, 576]")
    if kv_cache.shape[-1] != 656 or kv_cache.dim() not in (3, 4) or \
            (kv_cache.dim() == 4 and kv_cache.shape[2] != 1):
        raise ValueError("kv_cache must be [num_pages, page_size, 656] (or [.., .., 1, 656])")
    B, s_q, h_q, _ = q.shape
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(576)
    if out is None:
        out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device=device)
    else:
        _check("out", out, (torch.bfloat16,), device)
    if lse is None and return_lse:
        lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device=device)
    elif lse is not None:
        _check("lse", lse, (torch.float32,), device)
    dims = _decode_dims(B, s_q, h_q, indices.shape[2], kv_cache.shape[0], kv_cache.shape[1], softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    lib = load_library()
    if num_splits is None:
        status = lib.bsa_fp8_sparse_decode(
            _ptr(q), _ptr(kv_cache), _ptr(indices), ctypes.byref(dims), _ptr(out), _ptr(lse),
            ctypes.c_void_p(stream))
    else:
        if num_splits == "auto":
            num_splits = lib.bsa_fp8_sparse_decode_num_splits(ctypes.byref(dims))
        need = lib.bsa_fp8_sparse_decode_workspace_bytes(ctypes.byref(dims), int(num_splits))
        if need < 0:
            raise ValueError(f"num_splits={num_splits} is out of range")
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
        elif workspace is not None:
            _check("workspace", workspace, (torch.uint8,), device)
            if workspace.numel() < need:
                raise ValueError(f"workspace holds {workspace.numel()} bytes; {need} are needed")
        status = lib.bsa_fp8_sparse_decode_ex(
            _ptr(q), _ptr(kv_cache), _ptr(indices), ctypes.byref(dims), int(num_splits), _ptr(workspace),
            _ptr(out), _ptr(lse), ctypes.c_void_p(stream))
    if status != 0:
        raise BsaError(status, status_string(status))
    return out, lse


def bsa_fp8_sparse_decode(q, kv_cache, indices, *, softmax_scale=None, out=None, lse=None,
                          return_lse=True, stream=None):
    """Call the C entry point of the same name: FP8 sparse decode (MQA over a
    paged cache of 656-byte token rows).  q bf16 [B, s_q, h_q, 576]; kv_cache
    uint8 [num_pages, page_size, 656] (or with a kv-head axis of 1); indices
    int32 [B, s_q, topk] of cache rows (page * page_size + slot, -1 unused).
    Returns (out bf16 [B, s_q, h_q, 512], lse float32 [B, h_q, s_q])."""
    return _sparse_decode(q, kv_cache, indices, softmax_scale, out, lse, return_lse, stream, None, None)


def bsa_fp8_sparse_decode_ex(q, kv_cache, indices, *, num_splits="auto", workspace=None,
                             softmax_scale=None, out=None, lse=None, return_lse=True, stream=None):
    """Call the C entry point of the same name: the sparse decode with each
    index list cut into num_splits parts ("auto": the library's choice) and
    merged.  workspace: a uint8 device tensor of at least
    bsa_fp8_sparse_decode_workspace_bytes bytes, allocated here when None."""
    return _sparse_decode(q, kv_cache, indices, softmax_scale, out, lse, return_lse, stream, num_splits,
                          workspace)


def bsa_fp8_sparse_decode_noalloc(q, kv_cache, indices, out, lse, *, num_splits=0, softmax_scale=None,
                                  stream=None):
    """Call the C entry point of the same name: the split-list decode with its
    partial results in the library's static scratch, so nothing is allocated
    on the device by this call.  ``out`` (bf16 [B, s_q, h_q, 512]) and ``lse``
    (float32 [B, h_q, s_q] or None) are the caller's.  num_splits 0 = the
    library's choice within the scratch."""
    device = q.device
    if device.type != "cuda":
        raise ValueError("bsa_fp8_sparse_decode_noalloc runs on a GPU; q is on " + str(device))
    _check("q", q, (torch.bfloat16,), device)
    _check("kv_cache", kv_cache, (torch.uint8,), device)
    _check("indices", indices, (torch.int32,), device)
    _check("out", out, (torch.bfloat16,), device)
    if lse is not None:
        _check("lse", lse, (torch.float32,), device)
    if q.dim() != 4 or q.shape[3] != 576 or kv_cache.shape[-1] != 656:
        raise ValueError("q must be [B, s_q, h_q, 576] and kv_cache [num_pages, page_size, 656]")
    B, s_q, h_q, _ = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(576)
    dims = _decode_dims(B, s_q, h_q, indices.shape[2], kv_cache.shape[0], kv_cache.shape[1], softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    status = load_library().bsa_fp8_sparse_decode_noalloc(
        _ptr(q), _ptr(kv_cache), _ptr(indices), ctypes.byref(dims), int(num_splits), _ptr(out), _ptr(lse),
        ctypes.c_void_p(stream))
    if status != 0:
        raise BsaError(status, status_string(status))
    return out, lse


def attention_with_kvcache_blocksparse_prefill_fp8(
        q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_ids, seqlens_kvcache,
        max_seqlens_q, quant_type=QuantType.QPERTOKEN_PERHEAD_KPERTENSOR_VPERTENSOR,
        block_mask=None, kv_layout="NHD", softmax_scale=None, causal=True):
    """The call shape of the hpc-ops quick-start example (hpc-ops article,
    "Quick start"): page size comes from the cache shape, the layout is named
    by string, and the result is (out, lse)."""
    layout = KVLayout[kv_layout] if isinstance(kv_layout, str) else KVLayout(int(kv_layout))
    page_size = kcache.shape[1] if layout == KVLayout.NHD else kcache.shape[2]
    return bsa_fp8_prefill(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_ids,
                           seqlens_kvcache, block_mask, int(quant_type), page_size,
                           max_seqlen_q=max_seqlens_q, kv_layout=layout, causal=causal,
                           softmax_scale=softmax_scale)
