"""Python binding of the FP4 KV-cache C ABI (include/fp4kv.h).

Argument marshalling only: torch tensors are checked for dtype, device and
contiguity and handed to the HIP library as raw pointers on the current
stream; every step of the computation runs in the library's kernels.  If the
library has not been built this module raises instead of computing anything
another way.

    layout = cache_layout(num_kv_heads=8, head_dim=128, num_pages=n)
    cache = torch.empty(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    quantize_append(layout, k, v, slot_mapping, cache)
    out = decode_attention(layout, cache, q, seq_lens, page_table)
"""
import ctypes
import math
import os

__all__ = ["Fp4KVError", "CacheParams", "CacheLayout", "DecodePlan", "library", "cache_layout", "decode_plan",
           "quantize_append", "decode_attention", "decode_attention_noalloc", "decode_split", "decode_combine",
           "decode_append_attention", "decode_append_split", "decode_multi_attention",
           "decode_window_plan", "decode_window_attention", "DecodeOptions", "decode_with_options",
           "status_string", "PAGE_SIZE", "MAX_GROUP", "FORMAT_FP4_E2M1", "FORMAT_FP8_E4M3", "FORMAT_FP8_E4M3_TOKEN",
           "IntDims", "INT_PER_TOKEN", "INT_PER_CHANNEL", "INT_FP8_E4M3", "int_sizes", "int_quantize", "int_decode_plan",
           "int_decode_attention"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(HERE, "libfp4kv.so")
PAGE_SIZE = 64
MAX_GROUP = 16
NOALLOC_WORKSPACE_BYTES = 32 << 20   # the static workspace of decode_attention_noalloc
VERSION = 200                        # FP4KV_VERSION of the header these bindings follow
INT_PER_TOKEN = 0
INT_PER_CHANNEL = 1
INT_FP8_E4M3 = 0x108          # the `bits` value of FP8 E4M3 codes with fp16 scales

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5


class Fp4KVError(RuntimeError):
    def __init__(self, call, status):
        super().__init__(f"{call}: {status_string(status)} ({status})")
        self.status = status


FORMAT_FP4_E2M1 = 0        # E2M1 elements, one E4M3 scale per 16 channels
FORMAT_FP8_E4M3 = 1        # E4M3 elements, one fp32 scale per tensor
FORMAT_FP8_E4M3_TOKEN = 2  # E4M3 elements, one fp16 scale per (token, KV head)


class CacheParams(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("format", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


class CacheLayout(ctypes.Structure):
    _fields_ = [("params", CacheParams), ("block_bytes", ctypes.c_int64),
                ("k_codes_offset", ctypes.c_int64), ("k_scales_offset", ctypes.c_int64),
                ("v_codes_offset", ctypes.c_int64), ("v_scales_offset", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("page_stride", ctypes.c_int64),
                ("cache_bytes", ctypes.c_int64), ("bytes_per_token", ctypes.c_int64)]

    @property
    def num_kv_heads(self):
        return self.params.num_kv_heads

    @property
    def head_dim(self):
        return self.params.head_dim

    @property
    def num_pages(self):
        return self.params.num_pages

    @property
    def format(self):
        return self.params.format

    @property
    def fp8(self):
        return self.params.format in (FORMAT_FP8_E4M3, FORMAT_FP8_E4M3_TOKEN)

    @property
    def token_scales(self):
        return self.params.format == FORMAT_FP8_E4M3_TOKEN


class DecodeOptions(ctypes.Structure):
    """fp4kv_decode_options: the split kernel and how partials are merged."""
    _fields_ = [("kernel", ctypes.c_int32), ("merge", ctypes.c_int32), ("min_seq_len", ctypes.c_int32)]


DECODE_KERNELS = {"auto": 0, "mfma_staged": 1, "mfma_direct": 2, "valu": 3}
DECODE_MERGES = {"auto": 0, "combine_kernel": 1, "none": 2}

_LIB = None
_P = ctypes.c_void_p


class IntDims(ctypes.Structure):
    """fp4kv_int_dims: B sequences of T tokens, H KV heads of D channels."""
    _fields_ = [("batch", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


def library():
    """The loaded libfp4kv.so.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY_PATH):
            raise RuntimeError(f"{LIBRARY_PATH} is missing: build it with "
                               "`python -m fp4_quantised_kv_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIBRARY_PATH)
        L.fp4kv_version.argtypes = []
        L.fp4kv_version.restype = ctypes.c_int
        if L.fp4kv_version() != VERSION:
            raise RuntimeError(f"{LIBRARY_PATH} is version {L.fp4kv_version()}, these bindings follow {VERSION}: "
                               "rebuild it with `python -m fp4_quantised_kv_amd.build`")
        L.fp4kv_cache_layout.argtypes = [ctypes.POINTER(CacheParams), ctypes.POINTER(CacheLayout)]
        L.fp4kv_cache_layout.restype = ctypes.c_int
        L.fp4kv_quantize_append.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int64,
                                            _P, _P, _P]
        L.fp4kv_quantize_append.restype = ctypes.c_int
        L.fp4kv_decode_plan.argtypes = [ctypes.POINTER(CacheLayout), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
        L.fp4kv_decode_plan.restype = ctypes.c_int
        L.fp4kv_decode_attention.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int32,
                                             ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_float,
                                             ctypes.c_int32, _P, ctypes.c_int64, _P, _P]
        L.fp4kv_decode_attention.restype = ctypes.c_int
        L.fp4kv_decode_attention_noalloc.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int32,
                                                     ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_float,
                                                     ctypes.c_int32, _P, _P]
        L.fp4kv_decode_attention_noalloc.restype = ctypes.c_int
        L.fp4kv_decode_split.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_float,
                                         ctypes.c_int32, _P, ctypes.c_int64, _P]
        L.fp4kv_decode_split.restype = ctypes.c_int
        L.fp4kv_decode_combine.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _P, ctypes.c_int64, _P, _P]
        L.fp4kv_decode_combine.restype = ctypes.c_int
        L.fp4kv_decode_append_attention.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, _P, _P,
                                                    ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_int32, _P, ctypes.c_int64, _P, _P]
        L.fp4kv_decode_append_attention.restype = ctypes.c_int
        L.fp4kv_decode_append_split.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, _P, _P,
                                                ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                                ctypes.c_float, ctypes.c_int32, _P, ctypes.c_int64, _P]
        L.fp4kv_decode_append_split.restype = ctypes.c_int
        L.fp4kv_decode_multi_attention.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                                   ctypes.c_float, ctypes.c_int32, _P, ctypes.c_int64, _P, _P]
        L.fp4kv_decode_multi_attention.restype = ctypes.c_int
        L.fp4kv_decode_window_plan.argtypes = [ctypes.POINTER(CacheLayout), ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int64)]
        L.fp4kv_decode_window_plan.restype = ctypes.c_int
        L.fp4kv_decode_window_attention.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_float, ctypes.c_int32, _P,
                                                    ctypes.c_int64, _P, _P]
        L.fp4kv_decode_window_attention.restype = ctypes.c_int
        L.fp4kv_decode_with_options.argtypes = [ctypes.POINTER(CacheLayout), _P, _P, _P, _P, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_float, ctypes.c_int32, _P,
                                                ctypes.c_int64, _P, ctypes.POINTER(DecodeOptions), _P]
        L.fp4kv_decode_with_options.restype = ctypes.c_int
        L.fp4kv_read_probe.argtypes = [_P, ctypes.c_int64, _P, _P]
        L.fp4kv_read_probe.restype = ctypes.c_int
        L.fp4kv_read_probe_config.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              _P, _P]
        L.fp4kv_read_probe_config.restype = ctypes.c_int
        L.fp4kv_decode_chunks.argtypes = [ctypes.POINTER(CacheLayout), ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]
        L.fp4kv_decode_chunks.restype = ctypes.c_int
        L.fp4kv_stream_probe.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P]
        L.fp4kv_stream_probe.restype = ctypes.c_int
        L.fp4kv_int_sizes.argtypes = [ctypes.POINTER(IntDims), ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.fp4kv_int_sizes.restype = ctypes.c_int
        L.fp4kv_int_quantize.argtypes = [ctypes.POINTER(IntDims), ctypes.c_int32, ctypes.c_int32,
                                         _P, _P, _P, _P]
        L.fp4kv_int_quantize.restype = ctypes.c_int
        L.fp4kv_int_decode_plan.argtypes = [ctypes.POINTER(IntDims), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
        L.fp4kv_int_decode_plan.restype = ctypes.c_int
        L.fp4kv_int_decode_attention.argtypes = [ctypes.POINTER(IntDims), ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                 ctypes.c_float, ctypes.c_int32, _P, ctypes.c_int64,
                                                 _P, _P]
        L.fp4kv_int_decode_attention.restype = ctypes.c_int
        L.fp4kv_status_string.argtypes = [ctypes.c_int]
        L.fp4kv_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return library().fp4kv_status_string(int(status)).decode()


def _check(call, rc):
    if rc != OK:
        raise Fp4KVError(call, rc)


def cache_layout(num_kv_heads: int, head_dim: int, num_pages: int, page_size: int = PAGE_SIZE,
                 format: int = FORMAT_FP4_E2M1, k_scale: float = 0.0, v_scale: float = 0.0) -> CacheLayout:
    """Layout of a paged cache.  FP8 with per-tensor scales
    (format=FORMAT_FP8_E4M3) takes the K and V tensors' scales; FP4 and FP8
    with per-token scales (FORMAT_FP8_E4M3_TOKEN) take none (0)."""
    p = CacheParams(num_kv_heads, head_dim, page_size, format, num_pages, k_scale, v_scale)
    out = CacheLayout()
    _check("fp4kv_cache_layout", library().fp4kv_cache_layout(ctypes.byref(p), ctypes.byref(out)))
    return out


class DecodePlan(tuple):
    """(splits, partials, workspace_bytes) of fp4kv_decode_plan."""
    __slots__ = ()

    def __new__(cls, splits, partials, workspace_bytes):
        return tuple.__new__(cls, (splits, partials, workspace_bytes))

    splits = property(lambda self: self[0])
    partials = property(lambda self: self[1])
    workspace_bytes = property(lambda self: self[2])


_PLANS = {}


def decode_plan(layout: CacheLayout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                num_splits: int = 0) -> DecodePlan:
    """Context chunks, partials per row and workspace bytes that
    decode_attention uses for these arguments (the library's answer, kept per
    argument set: the plan is a pure function of them)."""
    key = (bytes(layout), batch, num_q_heads, max_pages_per_seq, num_splits)
    plan = _PLANS.get(key)
    if plan is None:
        plan = _PLANS[key] = _decode_plan(layout, batch, num_q_heads, max_pages_per_seq, num_splits)
    return plan


def _decode_plan(layout, batch, num_q_heads, max_pages_per_seq, num_splits):
    s = ctypes.c_int32()
    p = ctypes.c_int32()
    ws = ctypes.c_int64()
    _check("fp4kv_decode_plan", library().fp4kv_decode_plan(
        ctypes.byref(layout), batch, num_q_heads, max_pages_per_seq, num_splits,
        ctypes.byref(s), ctypes.byref(p), ctypes.byref(ws)))
    return DecodePlan(s.value, p.value, ws.value)


class DecodeChunks(tuple):
    """(lead_chunks, lead_pages, tail_pages) of fp4kv_decode_chunks: chunks
    0 .. lead_chunks - 1 hold lead_pages pages each, the later ones
    tail_pages each."""
    __slots__ = ()

    def __new__(cls, lead_chunks, lead_pages, tail_pages):
        return tuple.__new__(cls, (lead_chunks, lead_pages, tail_pages))

    lead_chunks = property(lambda self: self[0])
    lead_pages = property(lambda self: self[1])
    tail_pages = property(lambda self: self[2])

    def first_page(self, k: int) -> int:
        """First page (from the span's start) of chunk k."""
        if k < self.lead_chunks:
            return k * self.lead_pages
        return self.lead_chunks * self.lead_pages + (k - self.lead_chunks) * self.tail_pages


def decode_chunks(layout: CacheLayout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                  num_splits: int = 0, q_tokens: int = 1, window: int = 0, min_seq_len: int = 0) -> DecodeChunks:
    """Chunk page counts a decode call with these arguments uses
    (fp4kv_decode_chunks); min_seq_len as decode_with_options takes it."""
    lc, lp, tp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check("fp4kv_decode_chunks", library().fp4kv_decode_chunks(
        ctypes.byref(layout), batch, q_tokens, num_q_heads, max_pages_per_seq, window, num_splits, min_seq_len,
        ctypes.byref(lc), ctypes.byref(lp), ctypes.byref(tp)))
    return DecodeChunks(lc.value, lp.value, tp.value)


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t, name, dtype, device_type="cuda"):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != device_type:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_append(layout: CacheLayout, k, v, slot_mapping, cache, stream=None):
    """Quantise k, v (bf16 [n_tokens][H_kv][D]) into `cache` at `slot_mapping`
    (int64 [n_tokens]; negative slots are skipped)."""
    import torch
    for t, n, d in ((k, "k", torch.bfloat16), (v, "v", torch.bfloat16),
                    (slot_mapping, "slot_mapping", torch.int64), (cache, "cache", torch.uint8)):
        _need(t, n, d)
    n = k.shape[0] if k.dim() else 0
    want = (n, layout.num_kv_heads, layout.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must have shape {want}")
    if tuple(slot_mapping.shape) != (n,):
        raise ValueError("slot_mapping must have one entry per token")
    if cache.numel() < layout.cache_bytes:
        raise ValueError("cache is smaller than layout.cache_bytes")
    _check("fp4kv_quantize_append", library().fp4kv_quantize_append(
        ctypes.byref(layout), k.data_ptr(), v.data_ptr(), n, slot_mapping.data_ptr(),
        cache.data_ptr(), _stream(stream)))


def _decode_inputs(layout, cache, q, seq_lens, page_table, num_splits, workspace):
    import torch
    _need(cache, "cache", torch.uint8)
    _need(q, "q", torch.bfloat16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_table, "page_table", torch.int32)
    B, Hq, D = q.shape
    if D != layout.head_dim:
        raise ValueError("q's last dimension must equal the cache head_dim")
    if tuple(seq_lens.shape) != (B,) or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B][max_pages]")
    if cache.numel() < layout.cache_bytes:
        raise ValueError("cache is smaller than layout.cache_bytes")
    max_pages = page_table.shape[1]
    plan = decode_plan(layout, B, Hq, max_pages, num_splits)
    if workspace is None:
        workspace = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8)
    return B, Hq, D, max_pages, plan, workspace


def _out_tensor(out, B, Hq, D, device):
    import torch
    if out is None:
        return torch.empty(B, Hq, D, dtype=torch.float32, device=device)
    _need(out, "out", torch.float32)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    return out


def decode_attention(layout: CacheLayout, cache, q, seq_lens, page_table, softmax_scale=None,
                     num_splits: int = 0, workspace=None, out=None, stream=None):
    """Decode attention of q (bf16 [B][Hq][D]) over the cache; returns fp32
    [B][Hq][D].  seq_lens int32 [B]; page_table int32 [B][max_pages]."""
    B, Hq, D, max_pages, plan, workspace = _decode_inputs(
        layout, cache, q, seq_lens, page_table, num_splits, workspace)
    out = _out_tensor(out, B, Hq, D, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_attention", library().fp4kv_decode_attention(
        ctypes.byref(layout), cache.data_ptr(), q.data_ptr(), B, Hq, seq_lens.data_ptr(),
        page_table.data_ptr(), max_pages, float(softmax_scale), num_splits,
        workspace.data_ptr(), workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def decode_attention_noalloc(layout: CacheLayout, cache, q, seq_lens, page_table, softmax_scale=None,
                             num_splits: int = 0, out=None, stream=None):
    """decode_attention with the library's static workspace
    (NOALLOC_WORKSPACE_BYTES per GPU) instead of a caller's: the C call
    allocates nothing.  `out` (fp32 [B][Hq][D]) should be given by callers
    that must not allocate; without it this binding allocates the result."""
    import torch
    _need(cache, "cache", torch.uint8)
    _need(q, "q", torch.bfloat16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_table, "page_table", torch.int32)
    B, Hq, D = q.shape
    if D != layout.head_dim:
        raise ValueError("q's last dimension must equal the cache head_dim")
    if tuple(seq_lens.shape) != (B,) or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B][max_pages]")
    if cache.numel() < layout.cache_bytes:
        raise ValueError("cache is smaller than layout.cache_bytes")
    out = _out_tensor(out, B, Hq, D, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_attention_noalloc", library().fp4kv_decode_attention_noalloc(
        ctypes.byref(layout), cache.data_ptr(), q.data_ptr(), B, Hq, seq_lens.data_ptr(),
        page_table.data_ptr(), page_table.shape[1], float(softmax_scale), num_splits, out.data_ptr(),
        _stream(stream)))
    return out


def decode_split(layout: CacheLayout, cache, q, seq_lens, page_table, softmax_scale=None,
                 num_splits: int = 0, workspace=None, stream=None):
    """First half of decode_attention: per-workgroup partials in the
    workspace.  Returns (workspace, plan)."""
    B, Hq, D, max_pages, plan, workspace = _decode_inputs(
        layout, cache, q, seq_lens, page_table, num_splits, workspace)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_split", library().fp4kv_decode_split(
        ctypes.byref(layout), cache.data_ptr(), q.data_ptr(), B, Hq, seq_lens.data_ptr(),
        page_table.data_ptr(), max_pages, float(softmax_scale), num_splits,
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return workspace, plan


def decode_multi_attention(layout: CacheLayout, cache, q, seq_lens, page_table, softmax_scale=None,
                           num_splits: int = 0, workspace=None, out=None, stream=None):
    """Causal attention of several query tokens per sequence: q bf16
    [B][S][Hq][D] holds the last S positions of each context; query token i
    attends over the first seq_lens[b] - (S - 1 - i) tokens.  Returns fp32
    [B][S][Hq][D]."""
    import torch
    _need(cache, "cache", torch.uint8)
    _need(q, "q", torch.bfloat16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_table, "page_table", torch.int32)
    if q.dim() != 4:
        raise ValueError("q must be [B][S][Hq][D]")
    B, S, Hq, D = q.shape
    if D != layout.head_dim:
        raise ValueError("q's last dimension must equal the cache head_dim")
    if tuple(seq_lens.shape) != (B,) or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B][max_pages]")
    max_pages = page_table.shape[1]
    plan = decode_plan(layout, B, S * Hq, max_pages, num_splits)
    if workspace is None:
        workspace = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty(B, S, Hq, D, dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32)
        if tuple(out.shape) != (B, S, Hq, D):
            raise ValueError("out must be [B][S][Hq][D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_multi_attention", library().fp4kv_decode_multi_attention(
        ctypes.byref(layout), cache.data_ptr(), q.data_ptr(), B, S, Hq, seq_lens.data_ptr(),
        page_table.data_ptr(), max_pages, float(softmax_scale), num_splits, workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def decode_window_plan(layout: CacheLayout, batch: int, q_tokens: int, num_q_heads: int, max_pages_per_seq: int,
                       window: int, num_splits: int = 0) -> "DecodePlan":
    """Plan of a multi-query / sliding-window call (kept per argument set)."""
    key = ("window", bytes(layout), batch, q_tokens, num_q_heads, max_pages_per_seq, window, num_splits)
    plan = _PLANS.get(key)
    if plan is None:
        plan = _PLANS[key] = _decode_window_plan(layout, batch, q_tokens, num_q_heads, max_pages_per_seq, window,
                                                 num_splits)
    return plan


def _decode_window_plan(layout, batch, q_tokens, num_q_heads, max_pages_per_seq, window, num_splits):
    s, p, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check("fp4kv_decode_window_plan", library().fp4kv_decode_window_plan(
        ctypes.byref(layout), batch, q_tokens, num_q_heads, max_pages_per_seq, window, num_splits,
        ctypes.byref(s), ctypes.byref(p), ctypes.byref(ws)))
    return DecodePlan(s.value, p.value, ws.value)


def decode_window_attention(layout: CacheLayout, cache, q, seq_lens, page_table, window: int,
                            softmax_scale=None, num_splits: int = 0, workspace=None, out=None, stream=None):
    """Sliding-window causal attention: q bf16 [B][S][Hq][D] (the last S
    positions of each context); query token i sees the last `window` tokens
    of its prefix (window 0: all of it).  Returns fp32 [B][S][Hq][D]."""
    import torch
    _need(cache, "cache", torch.uint8)
    _need(q, "q", torch.bfloat16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_table, "page_table", torch.int32)
    if q.dim() != 4:
        raise ValueError("q must be [B][S][Hq][D]")
    B, S, Hq, D = q.shape
    if D != layout.head_dim:
        raise ValueError("q's last dimension must equal the cache head_dim")
    if tuple(seq_lens.shape) != (B,) or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B][max_pages]")
    max_pages = page_table.shape[1]
    plan = decode_window_plan(layout, B, S, Hq, max_pages, window, num_splits)
    if workspace is None:
        workspace = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty(B, S, Hq, D, dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32)
        if tuple(out.shape) != (B, S, Hq, D):
            raise ValueError("out must be [B][S][Hq][D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_window_attention", library().fp4kv_decode_window_attention(
        ctypes.byref(layout), cache.data_ptr(), q.data_ptr(), B, S, Hq, seq_lens.data_ptr(),
        page_table.data_ptr(), max_pages, int(window), float(softmax_scale), num_splits, workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def decode_with_options(layout: CacheLayout, cache, q, seq_lens, page_table, k_new=None, v_new=None, window=0,
                        softmax_scale=None, num_splits: int = 0, workspace=None, out=None, kernel="auto",
                        merge="auto", min_seq_len: int = 0, stream=None):
    """fp4kv_decode_with_options: any decode call with an explicit split
    kernel ("auto", "mfma_staged", "mfma_direct", "valu"), merge ("auto",
    "combine_kernel", or "none": the split kernel alone, returning
    (workspace, plan) as decode_split does) and min_seq_len (the host's lower
    bound on every seq_lens[b], 0 if unknown: it sizes the chunks only).  q
    is bf16 [B][Hq][D] (one query token; the result is [B][Hq][D]) or
    [B][S][Hq][D]; k_new, v_new (bf16 [B][H_kv][D]) append the step's token
    first (one query token, no window)."""
    import torch
    _need(cache, "cache", torch.uint8)
    _need(q, "q", torch.bfloat16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_table, "page_table", torch.int32)
    one = q.dim() == 3
    B, S, Hq, D = (q.shape[0], 1, q.shape[1], q.shape[2]) if one else tuple(q.shape)
    if D != layout.head_dim:
        raise ValueError("q's last dimension must equal the cache head_dim")
    if tuple(seq_lens.shape) != (B,) or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B][max_pages]")
    if cache.numel() < layout.cache_bytes:
        raise ValueError("cache is smaller than layout.cache_bytes")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _new_token_rows(layout, k_new, v_new, B)
    max_pages = page_table.shape[1]
    plan = decode_window_plan(layout, B, S, Hq, max_pages, window, num_splits)
    if workspace is None:
        workspace = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8)
    shape = (B, Hq, D) if one else (B, S, Hq, D)
    partials_only = merge == "none"
    if partials_only:
        if out is not None:
            raise ValueError("merge='none' writes no output rows: pass no out")
    elif out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {list(shape)}")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    opts = DecodeOptions(DECODE_KERNELS[kernel], DECODE_MERGES[merge], int(min_seq_len))
    ptr = lambda t: None if t is None else t.data_ptr()
    _check("fp4kv_decode_with_options", library().fp4kv_decode_with_options(
        ctypes.byref(layout), cache.data_ptr(), ptr(k_new), ptr(v_new), q.data_ptr(), B, S, Hq,
        seq_lens.data_ptr(), page_table.data_ptr(), max_pages, int(window), float(softmax_scale), num_splits,
        workspace.data_ptr(), workspace.numel(), ptr(out), ctypes.byref(opts), _stream(stream)))
    return (workspace, plan) if partials_only else out


def _new_token_rows(layout, k_new, v_new, B):
    import torch
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    want = (B, layout.num_kv_heads, layout.head_dim)
    if tuple(k_new.shape) != want or tuple(v_new.shape) != want:
        raise ValueError(f"k_new and v_new must have shape {want}")


def decode_append_attention(layout: CacheLayout, cache, k_new, v_new, q, seq_lens, page_table,
                            softmax_scale=None, num_splits: int = 0, workspace=None, out=None, stream=None):
    """One decode step with its own token: k_new, v_new (bf16 [B][H_kv][D])
    are stored at position seq_lens[b] - 1 of each sequence (seq_lens include
    the new token), then q attends over all seq_lens[b] tokens.  Returns fp32
    [B][Hq][D]."""
    B, Hq, D, max_pages, plan, workspace = _decode_inputs(
        layout, cache, q, seq_lens, page_table, num_splits, workspace)
    _new_token_rows(layout, k_new, v_new, B)
    out = _out_tensor(out, B, Hq, D, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_append_attention", library().fp4kv_decode_append_attention(
        ctypes.byref(layout), cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), B, Hq,
        seq_lens.data_ptr(), page_table.data_ptr(), max_pages, float(softmax_scale), num_splits,
        workspace.data_ptr(), workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def decode_append_split(layout: CacheLayout, cache, k_new, v_new, q, seq_lens, page_table,
                        softmax_scale=None, num_splits: int = 0, workspace=None, stream=None):
    """decode_append_attention without the combine: returns (workspace,
    plan) as decode_split does."""
    B, Hq, D, max_pages, plan, workspace = _decode_inputs(
        layout, cache, q, seq_lens, page_table, num_splits, workspace)
    _new_token_rows(layout, k_new, v_new, B)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _check("fp4kv_decode_append_split", library().fp4kv_decode_append_split(
        ctypes.byref(layout), cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), B, Hq,
        seq_lens.data_ptr(), page_table.data_ptr(), max_pages, float(softmax_scale), num_splits,
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return workspace, plan


def decode_combine(workspace, batch: int, num_q_heads: int, head_dim: int, partials: int,
                   out=None, stream=None):
    """Second half of decode_attention: merge `partials` partial results per
    row into fp32 [batch][num_q_heads][head_dim]."""
    import torch
    _need(workspace, "workspace", torch.uint8)
    out = _out_tensor(out, batch, num_q_heads, head_dim, workspace.device)
    _check("fp4kv_decode_combine", library().fp4kv_decode_combine(
        batch, num_q_heads, head_dim, partials, workspace.data_ptr(), workspace.numel(),
        out.data_ptr(), _stream(stream)))
    return out


def read_probe(buf, sink, stream=None):
    """Measurement utility: stream `buf` (uint8, a multiple of 9216 bytes) once
    through 16-byte loads and discard it; `sink` is a 4-byte device tensor."""
    import torch
    _need(buf, "buf", torch.uint8)
    _need(sink, "sink", torch.int32)
    _check("fp4kv_read_probe", library().fp4kv_read_probe(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                                                          _stream(stream)))


def read_probe_config(buf, sink, loads_per_lane: int, workgroups: int, to_lds: bool = False, stream=None):
    """Measurement utility: the read probe with a chosen shape (see
    fp4kv_read_probe_config); `buf` uint8, a multiple of 1024 * loads_per_lane
    bytes."""
    import torch
    _need(buf, "buf", torch.uint8)
    _need(sink, "sink", torch.int32)
    _check("fp4kv_read_probe_config", library().fp4kv_read_probe_config(
        buf.data_ptr(), buf.numel(), int(loads_per_lane), int(workgroups), int(bool(to_lds)), sink.data_ptr(),
        _stream(stream)))


def stream_probe(src, dst, read_bytes: int, write_bytes: int, paired: bool, workgroups: int, sink, stream=None):
    """Measurement utility: streaming reads and writes in a given proportion
    (fp4kv_stream_probe); units = src.numel() // read_bytes, and dst must
    hold units * write_bytes bytes."""
    import torch
    _need(src, "src", torch.uint8)
    _need(dst, "dst", torch.uint8)
    _need(sink, "sink", torch.int32)
    units = src.numel() // read_bytes
    if units < 1 or dst.numel() < units * write_bytes:
        raise ValueError("stream_probe: src must hold a unit and dst units * write_bytes bytes")
    _check("fp4kv_stream_probe", library().fp4kv_stream_probe(
        src.data_ptr(), dst.data_ptr(), units, int(read_bytes), int(write_bytes), int(bool(paired)), int(workgroups),
        sink.data_ptr(), _stream(stream)))


# ------------------------------------------- integer formats (include/fp4kv_int.h)

def _gran(g):
    return {"token": INT_PER_TOKEN, "channel": INT_PER_CHANNEL}.get(g, g)


def _element_bits(bits: int) -> int:
    return 8 if bits == INT_FP8_E4M3 else int(bits)


def int_sizes(batch: int, tokens: int, num_kv_heads: int, head_dim: int, bits: int, granularity="token"):
    """(code bytes, scale bytes) of one tensor in a sweep format (bits 2, 4, 8,
    INT_FP8_E4M3, or 16 for the unquantised bf16 copy)."""
    d = IntDims(batch, tokens, num_kv_heads, head_dim)
    c, s = ctypes.c_int64(), ctypes.c_int64()
    _check("fp4kv_int_sizes", library().fp4kv_int_sizes(ctypes.byref(d), int(bits), _gran(granularity),
                                                        ctypes.byref(c), ctypes.byref(s)))
    return c.value, s.value


def int_quantize(x, bits: int, granularity="token", stream=None):
    """Quantise x (bf16 [B][T][H][D]) to symmetric bits-bit integer codes, or
    to E4M3 codes for bits = INT_FP8_E4M3, with fp16 scales per token or per
    channel.  Returns (codes uint8 [B][H][T][D * element bits / 8], scales
    int16 fp16 bit patterns: [B][H][T] per token, [B][H][D] per channel,
    empty for bits 16)."""
    import torch
    _need(x, "x", torch.bfloat16)
    if x.dim() != 4:
        raise ValueError("x must be [B][T][H][D]")
    B, T, H, D = x.shape
    d = IntDims(B, T, H, D)
    nc, ns = int_sizes(B, T, H, D, bits, granularity)
    codes = torch.empty(max(nc, 16), dtype=torch.uint8, device=x.device)
    scales = torch.empty(max(ns // 2, 8), dtype=torch.int16, device=x.device)
    _check("fp4kv_int_quantize", library().fp4kv_int_quantize(
        ctypes.byref(d), int(bits), _gran(granularity), x.data_ptr(), codes.data_ptr(),
        scales.data_ptr(), _stream(stream)))
    codes = codes[:nc].view(B, H, T, D * _element_bits(bits) // 8)
    if bits == 16:
        scales = scales[:0]
    elif _gran(granularity) == INT_PER_TOKEN:
        scales = scales[: ns // 2].view(B, H, T)
    else:
        scales = scales[: ns // 2].view(B, H, D)
    return codes, scales


def int_decode_plan(batch: int, tokens: int, num_kv_heads: int, head_dim: int, num_q_heads: int,
                    num_splits: int = 0):
    """(splits, workspace bytes) of int_decode_attention."""
    d = IntDims(batch, tokens, num_kv_heads, head_dim)
    s, ws = ctypes.c_int32(), ctypes.c_int64()
    _check("fp4kv_int_decode_plan", library().fp4kv_int_decode_plan(
        ctypes.byref(d), num_q_heads, num_splits, ctypes.byref(s), ctypes.byref(ws)))
    return s.value, ws.value


def int_decode_attention(q, bits: int, k, v, tokens: int, k_granularity="token", v_granularity="token",
                         softmax_scale=None, num_splits: int = 0, workspace=None, out=None, stream=None):
    """Decode attention of q (bf16 [B][Hq][D]) over K and V in a sweep format
    (integer, FP8 with fp16 scales, or bf16): k and v are the (codes, scales) pairs int_quantize returns for
    [B][tokens][H][D] tensors.  Returns fp32 [B][Hq][D]."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    (kc, ks), (vc, vs) = k, v
    for t, n in ((kc, "k codes"), (vc, "v codes")):
        _need(t, n, torch.uint8)
    for t, n in ((ks, "k scales"), (vs, "v scales")):
        _need(t, n, torch.int16)
    H = kc.shape[1]
    d = IntDims(B, tokens, H, D)
    for (c, sc), g in ((k, k_granularity), (v, v_granularity)):
        nc, ns = int_sizes(B, tokens, H, D, bits, g)
        if c.numel() != nc or sc.numel() * 2 != ns:
            raise ValueError("codes or scales do not match the dims, bits and granularity")
    splits, ws_bytes = int_decode_plan(B, tokens, H, D, Hq, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8)
    out = _out_tensor(out, B, Hq, D, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    ptr = lambda t: t.data_ptr() if t.numel() else None
    _check("fp4kv_int_decode_attention", library().fp4kv_int_decode_attention(
        ctypes.byref(d), int(bits), _gran(k_granularity), _gran(v_granularity), ptr(kc), ptr(ks),
        ptr(vc), ptr(vs), q.data_ptr(), Hq, float(softmax_scale), num_splits, workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), _stream(stream)))
    return out
