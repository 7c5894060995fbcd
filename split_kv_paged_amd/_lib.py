"""ctypes binding of libskv.so (include/skv.h), with the same function names.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in libskv's kernels.
Loading fails loudly when the library has not been built — there is no
fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskv.so")

SKV_OK, SKV_EINVAL, SKV_EUNSUPPORTED, SKV_ELAUNCH = 0, 1, 2, 3
LAYOUT = {"standard": 0, "shuffled": 1}
CONVERT_DIR = {"to_shuffled": 0, "to_standard": 1}
KV_DTYPE = {"bf16": 0, "fp8": 1, "fp16": 2}
ATTN_CLAIM_UNITS = 2              # flag of the attention entry points (fp8: run-time order)


def io_dtype(kv_dtype):
    """torch dtype of q and of the output: fp16 with an fp16 cache, else bf16."""
    return torch.float16 if kv_dtype == "fp16" else torch.bfloat16

_c_int, _c_sz, _p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "skv_plan_words": (_c_sz, [_c_int, _c_int, _c_int]),
    "skv_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int, _c_int]),
    "skv_plan_build": (_c_int, [_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _c_int, _p, _p, _p]),
    "skv_paged_decode_attn": (_c_int, [_p, _p, _p, _c_int, _c_int, _p, _c_int, _p, _p,
                                       _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _p, _p, _c_int, _p, _p, _c_int, _c_int,
                                       _p, _p, _p, _p, _c_int, _p]),
    "skv_segment_attn": (_c_int, [_p, _p, _p, _c_int, _c_int, _p, _c_int, _p, _p,
                                  _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _p, _p, _c_int, _p, _p, _c_int, _c_int,
                                  _p, _p, _c_int, _p]),
    "skv_split_reduce": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p,
                                  _p]),
    "skv_kv_page_shuffle": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _p]),
    "skv_kv_page_convert": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _p]),
    "skv_kv_page_unshuffle": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _p]),
    "skv_kv_cache_write": (_c_int, [_p, _p, _p, _c_int, ctypes.c_longlong, ctypes.c_longlong,
                                    _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p,
                                    _p]),
    "skv_paged_decode_attn_static": (_c_int, [_p, _p, _p, _c_int, _c_int, _p, _c_int, _p, _p,
                                              _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                              _c_int, _p, _p, _c_int, _p, _p, _c_int, _c_int,
                                              _p, _p, _c_int, _p]),
    "skv_check_inputs": (_c_int, [_p, _c_int, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _p, _p]),
    "skv_strerror": (ctypes.c_char_p, [_c_int]),
}
EXPORTED = tuple(_SIGNATURES)

_lib = None


class SkvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)})")


def load():
    """Load libskv.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m split_kv_paged_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def strerror(status):
    return load().skv_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != SKV_OK:
        raise SkvError(status, where)


def _need(t, dtype, name, numel=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs {numel} elements, has {t.numel()}")


def plan_words(bs, kv_heads, num_cus):
    return int(load().skv_plan_words(bs, kv_heads, num_cus))


def workspace_bytes(total_q, q_heads, head_dim, seg_max):
    return int(load().skv_workspace_bytes(total_q, q_heads, head_dim, seg_max))


def plan_build(seq_lens, cu_seqlens_q, total_q, kv_heads, num_cus, seg_max, causal=1,
               page_size=16, plan=None, tok_nseg=None, stream=None):
    """Enqueue the planner; returns (plan int32 [plan_words], tok_nseg int32 [total_q]).

    total_q is a host integer (cu_seqlens_q[-1]) so that nothing is read back."""
    bs = seq_lens.numel()
    dev = seq_lens.device
    if plan is None:
        plan = torch.empty(plan_words(bs, kv_heads, num_cus), dtype=torch.int32, device=dev)
    if tok_nseg is None:
        tok_nseg = torch.empty(max(total_q, 1), dtype=torch.int32, device=dev)
    _need(seq_lens, torch.int32, "seq_lens")
    _need(cu_seqlens_q, torch.int32, "cu_seqlens_q", bs + 1)
    _need(plan, torch.int32, "plan", plan_words(bs, kv_heads, num_cus))
    _need(tok_nseg, torch.int32, "tok_nseg")
    st = load().skv_plan_build(_ptr(seq_lens), _ptr(cu_seqlens_q), bs, total_q, kv_heads,
                               page_size, num_cus, seg_max, int(causal), _ptr(plan),
                               _ptr(tok_nseg), _stream(stream))
    _check(st, "skv_plan_build")
    return plan, tok_nseg


def paged_decode_attn(q, kv_a, kv_b, page_table, seq_lens, cu_seqlens_q, plan, tok_nseg,
                      *, kv_heads, max_q, num_cus, seg_max, kv_dtype="bf16",
                      layout="standard", k_scale=None, v_scale=None, causal=1,
                      part_o=None, part_lse=None, out=None, out_lse=None,
                      page_size=16, claim_units=False, stream=None):
    """Enqueue segment attention + split reduce; returns (out, out_lse or None);
    q and out are fp16 with kv_dtype="fp16", else bf16.

    plan=None selects the fixed split (no plan launch); tok_nseg is then
    written by the segment kernel (allocated when None). By default the
    summation order is fixed (bit-identical results for identical inputs);
    claim_units=True passes SKV_ATTN_CLAIM_UNITS (fp8 KV: run-time order,
    results agree to rounding)."""
    total_q, q_heads, head_dim = q.shape
    bs = seq_lens.numel()
    dev = q.device
    if plan is None and tok_nseg is None:
        tok_nseg = torch.empty(total_q, dtype=torch.int32, device=dev)
    rows = total_q * q_heads * seg_max
    if part_o is None:
        part_o = torch.empty(rows * head_dim, dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty(rows, dtype=torch.float32, device=dev)
    iot = io_dtype(kv_dtype)
    if out is None:
        out = torch.empty((total_q, q_heads, head_dim), dtype=iot, device=dev)
    _need(q, iot, "q")
    _need(out, iot, "out", total_q * q_heads * head_dim)
    _need(part_o, torch.float32, "part_o", rows * head_dim)
    _need(part_lse, torch.float32, "part_lse", rows)
    _need(page_table, torch.int32, "page_table")
    if plan is not None:
        _need(plan, torch.int32, "plan", plan_words(bs, kv_heads, num_cus))
    _need(tok_nseg, torch.int32, "tok_nseg", total_q)
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", total_q * q_heads)
    for t, n in ((kv_a, "kv_a"), (kv_b, "kv_b")):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{n}: expected a contiguous device tensor")
    st = load().skv_paged_decode_attn(
        _ptr(q), _ptr(kv_a), _ptr(kv_b), LAYOUT[layout], KV_DTYPE[kv_dtype],
        _ptr(page_table), page_table.shape[1], _ptr(seq_lens), _ptr(cu_seqlens_q), bs,
        total_q, max_q, q_heads, kv_heads, head_dim, page_size, _ptr(k_scale),
        _ptr(v_scale), int(causal), _ptr(plan), _ptr(tok_nseg), num_cus, seg_max,
        _ptr(part_o), _ptr(part_lse), _ptr(out), _ptr(out_lse),
        ATTN_CLAIM_UNITS if claim_units else 0, _stream(stream))
    _check(st, "skv_paged_decode_attn")
    return out, out_lse


def segment_attn(q, kv_a, kv_b, page_table, seq_lens, cu_seqlens_q, plan, tok_nseg,
                 *, kv_heads, max_q, num_cus, seg_max, part_o, part_lse, kv_dtype="bf16",
                 layout="standard", k_scale=None, v_scale=None, causal=1, page_size=16,
                 claim_units=False, stream=None):
    """Enqueue the segment kernel alone (partials only). plan=None: fixed split,
    tok_nseg written (allocated when None); returns (part_o, part_lse, tok_nseg)."""
    total_q, q_heads, head_dim = q.shape
    bs = seq_lens.numel()
    if plan is None and tok_nseg is None:
        tok_nseg = torch.empty(total_q, dtype=torch.int32, device=q.device)
    rows = total_q * q_heads * seg_max
    _need(q, io_dtype(kv_dtype), "q")
    _need(part_o, torch.float32, "part_o", rows * head_dim)
    _need(part_lse, torch.float32, "part_lse", rows)
    _need(page_table, torch.int32, "page_table")
    if plan is not None:
        _need(plan, torch.int32, "plan", plan_words(bs, kv_heads, num_cus))
    _need(tok_nseg, torch.int32, "tok_nseg", total_q)
    st = load().skv_segment_attn(
        _ptr(q), _ptr(kv_a), _ptr(kv_b), LAYOUT[layout], KV_DTYPE[kv_dtype],
        _ptr(page_table), page_table.shape[1], _ptr(seq_lens), _ptr(cu_seqlens_q), bs,
        total_q, max_q, q_heads, kv_heads, head_dim, page_size, _ptr(k_scale),
        _ptr(v_scale), int(causal), _ptr(plan), _ptr(tok_nseg), num_cus, seg_max,
        _ptr(part_o), _ptr(part_lse), ATTN_CLAIM_UNITS if claim_units else 0,
        _stream(stream))
    _check(st, "skv_segment_attn")
    return part_o, part_lse, tok_nseg


def split_reduce(part_o, part_lse, tok_nseg, *, total_q, q_heads, seg_max, head_dim=128,
                 out=None, out_lse=None, out_dtype="bf16", stream=None):
    """LSE merge of the partials; out bf16 (out_dtype "bf16") or fp16 ("fp16")."""
    dev = part_o.device
    iot = io_dtype(out_dtype)
    if out is None:
        out = torch.empty((total_q, q_heads, head_dim), dtype=iot, device=dev)
    rows = total_q * q_heads * seg_max
    _need(part_o, torch.float32, "part_o", rows * head_dim)
    _need(part_lse, torch.float32, "part_lse", rows)
    _need(tok_nseg, torch.int32, "tok_nseg", total_q)
    _need(out, iot, "out", total_q * q_heads * head_dim)
    st = load().skv_split_reduce(_ptr(part_o), _ptr(part_lse), _ptr(tok_nseg), total_q,
                                 q_heads, head_dim, seg_max, KV_DTYPE[out_dtype], _ptr(out),
                                 _ptr(out_lse), _stream(stream))
    _check(st, "skv_split_reduce")
    return out, out_lse


def kv_page_shuffle(std_cache, k_plane=None, v_plane=None, block_ids=None, stream=None):
    """Standard pages [B, H, N, 2D] -> (K plane [B, H, D/x, N, x], V plane [B, H, N/x, D, x])."""
    B, H, N, D2 = std_cache.shape
    D = D2 // 2
    e = std_cache.element_size()
    x = 16 // e
    if k_plane is None:
        k_plane = torch.empty((B, H, D // x, N, x), dtype=std_cache.dtype, device=std_cache.device)
    if v_plane is None:
        v_plane = torch.empty((B, H, N // x, D, x), dtype=std_cache.dtype, device=std_cache.device)
    for t, n in ((std_cache, "std_cache"), (k_plane, "k_plane"), (v_plane, "v_plane")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous device tensor")
    nb = B
    if block_ids is not None:
        _need(block_ids, torch.int32, "block_ids")
        nb = block_ids.numel()
    st = load().skv_kv_page_shuffle(_ptr(std_cache), _ptr(k_plane), _ptr(v_plane),
                                    _ptr(block_ids), nb, H, N, D, e, _stream(stream))
    _check(st, "skv_kv_page_shuffle")
    return k_plane, v_plane


def _planes(k_plane, v_plane):
    for t, n in ((k_plane, "k_plane"), (v_plane, "v_plane")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous device tensor")
    if k_plane.dim() != 5 or v_plane.dim() != 5:
        raise ValueError("planes: expected [B, H, D/x, N, x] and [B, H, N/x, D, x]")
    B, H, Dx, N, x = k_plane.shape
    if tuple(v_plane.shape) != (B, H, N // x, Dx * x, x) or v_plane.dtype != k_plane.dtype:
        raise ValueError("v_plane: shape or dtype does not match k_plane")
    return B, H, Dx * x, N, k_plane.element_size()


def kv_page_convert(k_plane, v_plane, block_ids=None, direction="to_shuffled", stream=None):
    """In place: K/V-plane blocks holding a standard block's two byte halves ->
    its shuffled K and V ("to_shuffled"), or back ("to_standard")."""
    B, H, D, N, e = _planes(k_plane, v_plane)
    nb = B
    if block_ids is not None:
        _need(block_ids, torch.int32, "block_ids")
        nb = block_ids.numel()
    st = load().skv_kv_page_convert(_ptr(k_plane), _ptr(v_plane), _ptr(block_ids), nb, H, N,
                                    D, e, CONVERT_DIR[direction], _stream(stream))
    _check(st, "skv_kv_page_convert")
    return k_plane, v_plane


def kv_page_unshuffle(k_plane, v_plane, std_cache=None, block_ids=None, stream=None):
    """Shuffled planes -> standard pages [B, H, N, 2D] (inverse of kv_page_shuffle)."""
    B, H, D, N, e = _planes(k_plane, v_plane)
    if std_cache is None:
        std_cache = torch.empty((B, H, N, 2 * D), dtype=k_plane.dtype, device=k_plane.device)
    if not std_cache.is_cuda or not std_cache.is_contiguous():
        raise ValueError("std_cache: expected a contiguous device tensor")
    nb = B
    if block_ids is not None:
        _need(block_ids, torch.int32, "block_ids")
        nb = block_ids.numel()
    st = load().skv_kv_page_unshuffle(_ptr(k_plane), _ptr(v_plane), _ptr(std_cache),
                                      _ptr(block_ids), nb, H, N, D, e, _stream(stream))
    _check(st, "skv_kv_page_unshuffle")
    return std_cache


def kv_cache_write(key, value, slot_mapping, k_plane, v_plane, k_scale=None, v_scale=None,
                   stream=None):
    """Write new tokens (key, value [T, H, D]; token rows may be strided) into
    the shuffled planes at slot_mapping (int64 [T]; negative = padding).
    Without scales key/value are in the cache's element type and copied; with
    k_scale/v_scale (fp32 [1] device tensors) they are bf16 and quantised into
    an fp8 cache. Returns the planes."""
    B, H, D, N, e = _planes(k_plane, v_plane)
    in_e = 2 if k_scale is not None else e
    for t, n in ((key, "key"), (value, "value")):
        if not t.is_cuda or t.dim() != 3 or t.shape[1:] != (H, D):
            raise ValueError(f"{n}: expected a device tensor [T, {H}, {D}]")
        if t.stride(2) != 1 or t.stride(1) != D or t.element_size() != in_e:
            raise ValueError(f"{n}: heads and channels must be dense, element size {in_e}")
    _need(slot_mapping, torch.int64, "slot_mapping", key.shape[0])
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is not None:
            _need(t, torch.float32, n, 1)
    T = key.shape[0]
    st = load().skv_kv_cache_write(_ptr(key), _ptr(value), _ptr(slot_mapping), T,
                                   key.stride(0), value.stride(0), _ptr(k_plane),
                                   _ptr(v_plane), B, H, N, D, e, _ptr(k_scale),
                                   _ptr(v_scale), _stream(stream))
    _check(st, "skv_kv_cache_write")
    return k_plane, v_plane


STATIC_SCRATCH_BYTES = 64 << 20      # SKV_STATIC_SCRATCH_BYTES


def paged_decode_attn_static(q, kv_a, kv_b, page_table, seq_lens, cu_seqlens_q, plan, tok_nseg,
                             *, kv_heads, max_q, num_cus, seg_max, kv_dtype="bf16",
                             layout="standard", k_scale=None, v_scale=None, causal=1,
                             out=None, out_lse=None, page_size=16, claim_units=False,
                             stream=None):
    """paged_decode_attn with the partials in the library's own device array
    (no workspace arguments; the library allocates nothing). Calls that
    overlap on one GPU race. Returns (out, out_lse or None)."""
    total_q, q_heads, head_dim = q.shape
    bs = seq_lens.numel()
    dev = q.device
    if plan is None and tok_nseg is None:
        tok_nseg = torch.empty(total_q, dtype=torch.int32, device=dev)
    iot = io_dtype(kv_dtype)
    if out is None:
        out = torch.empty((total_q, q_heads, head_dim), dtype=iot, device=dev)
    _need(q, iot, "q")
    _need(out, iot, "out", total_q * q_heads * head_dim)
    _need(page_table, torch.int32, "page_table")
    if plan is not None:
        _need(plan, torch.int32, "plan", plan_words(bs, kv_heads, num_cus))
    _need(tok_nseg, torch.int32, "tok_nseg", total_q)
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", total_q * q_heads)
    for t, n in ((kv_a, "kv_a"), (kv_b, "kv_b")):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{n}: expected a contiguous device tensor")
    st = load().skv_paged_decode_attn_static(
        _ptr(q), _ptr(kv_a), _ptr(kv_b), LAYOUT[layout], KV_DTYPE[kv_dtype],
        _ptr(page_table), page_table.shape[1], _ptr(seq_lens), _ptr(cu_seqlens_q), bs,
        total_q, max_q, q_heads, kv_heads, head_dim, page_size, _ptr(k_scale),
        _ptr(v_scale), int(causal), _ptr(plan), _ptr(tok_nseg), num_cus, seg_max,
        _ptr(out), _ptr(out_lse), ATTN_CLAIM_UNITS if claim_units else 0, _stream(stream))
    _check(st, "skv_paged_decode_attn_static")
    return out, out_lse


# bits of check_inputs' first result word (enum skv_contract_violation)
CONTRACT_BITS = {"len_negative": 1, "len_table": 2, "cu": 4, "qlen": 8, "page_id": 16}


def check_inputs(page_table, seq_lens, cu_seqlens_q, total_q, max_q, num_blocks, page_size=16,
                 result=None, stream=None):
    """Enqueue the device-data contract check; returns the int32 [2] device
    tensor it writes: [violation bits (CONTRACT_BITS), first offending
    sequence or -1]. Read it after the stream's work is done."""
    bs = seq_lens.numel()
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=seq_lens.device)
    _need(page_table, torch.int32, "page_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(cu_seqlens_q, torch.int32, "cu_seqlens_q", bs + 1)
    _need(result, torch.int32, "result", 2)
    if page_table.dim() != 2 or page_table.shape[0] < bs:
        raise ValueError("page_table: expected [bs, pt_stride]")
    st = load().skv_check_inputs(_ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                                 _ptr(cu_seqlens_q), bs, total_q, max_q, page_size, num_blocks,
                                 _ptr(result), _stream(stream))
    _check(st, "skv_check_inputs")
    return result
