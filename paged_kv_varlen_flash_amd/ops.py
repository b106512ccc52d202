"""ctypes binding of libpagedattn (declared in include/pagedattn.h).

The ``pa_*`` functions mirror the C entry points one to one and only
marshal arguments: tensors become device pointers, the current torch
stream becomes the HIP stream, C status codes become ``PaError``.  Every
computation runs in the library's HIP kernels (or, for the planner, in its
host C++).  There is no fallback: if ``libpagedattn.so`` is missing or a
tensor is not on the GPU, the call raises.

``VarlenPlan``/``plan_varlen``, ``varlen_fwd`` and ``cascade_fwd`` are
conveniences over the same calls: they size and allocate the device work
list and workspace with torch and upload the planner's output.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same library (for instance one whose
# host code is compiled with sanitizers); by default the in-tree build
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_HIP = 4
PA_WORKLIST_MAGIC = 0x50414731
PA_WORKLIST_HEADER_WORDS = 16
PA_ITEM_WORDS = 12
PA_TILED_ROWS = 128             # tiled item rows in launches with small-row items, or at D = 256
PA_TILED_ROWS_WIDE = 256        # tiled item rows otherwise
PLAN_TARGET_CUS = 256          # compute units the planner schedules for (PA_PLAN_TARGET_CUS)

EXPORTED = ["pa_status_str", "pa_version", "pa_supported_head_sizes", "pa_plan_varlen",
            "pa_cascade_split", "pa_reshape_and_cache", "pa_varlen_fwd", "pa_merge_attn_states",
            "pa_reshape_and_cache_fp8", "pa_varlen_fwd_fp8", "pa_cascade_decide",
            "pa_varlen_fwd_ex", "pa_varlen_fwd_noalloc", "pa_upload_words"]
NOALLOC_SCRATCH_BYTES = 32 << 20   # PA_NOALLOC_SCRATCH_BYTES


class PaError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class AttnParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("block_table_stride", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("sliding_window", ctypes.c_int32), ("kv_cache_fp8", ctypes.c_int32),
                ("num_cus", ctypes.c_int32)]

    def __repr__(self):
        return "AttnParams(" + ", ".join(f"{k}={getattr(self, k)}" for k, _ in self._fields_) + ")"


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_small_items", ctypes.c_int32), ("num_tiled_items", ctypes.c_int32),
                ("num_reduce_items", ctypes.c_int32), ("num_partial_rows", ctypes.c_int32),
                ("max_reduce_rows", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32), ("tiled_rows", ctypes.c_int32),
                ("worklist_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


PA_KV_BF16, PA_KV_E4M3 = 0, 1


class FwdOptions(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("s_aux", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_varlen_flash_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.pa_status_str.restype = ctypes.c_char_p
        L.pa_status_str.argtypes = [ctypes.c_int]
        L.pa_version.restype = ctypes.c_int32
        L.pa_plan_varlen.restype = ctypes.c_int
        L.pa_plan_varlen.argtypes = [ctypes.POINTER(AttnParams), _I32P, _I32P, ctypes.c_int32,
                                     _I32P, ctypes.c_size_t, ctypes.POINTER(PlanInfo)]
        L.pa_cascade_split.restype = ctypes.c_int
        L.pa_cascade_split.argtypes = [ctypes.POINTER(AttnParams), ctypes.c_int32, _I32P, _I32P,
                                       ctypes.POINTER(AttnParams), ctypes.POINTER(AttnParams),
                                       _I32P, _I32P, _I32P, _I32P]
        L.pa_cascade_decide.restype = ctypes.c_int
        L.pa_cascade_decide.argtypes = [ctypes.POINTER(AttnParams), _I32P, _I32P, _I32P,
                                        ctypes.c_int32, _I32P, _I32P]
        L.pa_reshape_and_cache.restype = ctypes.c_int
        L.pa_reshape_and_cache.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, _P]
        L.pa_varlen_fwd.restype = ctypes.c_int
        L.pa_varlen_fwd.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(PlanInfo), _P,
                                    _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                    ctypes.c_size_t, _P]
        L.pa_reshape_and_cache_fp8.restype = ctypes.c_int
        L.pa_reshape_and_cache_fp8.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                               _P, _P, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
        L.pa_varlen_fwd_fp8.restype = ctypes.c_int
        L.pa_varlen_fwd_fp8.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(PlanInfo), _P,
                                        _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                        ctypes.c_size_t, _P]
        L.pa_varlen_fwd_ex.restype = ctypes.c_int
        L.pa_varlen_fwd_ex.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(PlanInfo), _P,
                                       _P, _P, _P, _P, _P, ctypes.POINTER(FwdOptions),
                                       ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]
        L.pa_varlen_fwd_noalloc.restype = ctypes.c_int
        L.pa_varlen_fwd_noalloc.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(PlanInfo),
                                            _P, _P, _P, _P, _P, _P, ctypes.POINTER(FwdOptions),
                                            ctypes.c_int32, _P, _P, _P]
        L.pa_upload_words.restype = ctypes.c_int
        L.pa_upload_words.argtypes = [_P, _P, ctypes.c_int64, _P]
        L.pa_merge_attn_states.restype = ctypes.c_int
        L.pa_merge_attn_states.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _P]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().pa_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != PA_OK:
        raise PaError(status, where)


def supported_head_sizes():
    arr = (ctypes.c_int32 * 3).in_dll(lib(), "pa_supported_head_sizes")
    return list(arr)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr_i32(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_I32P)


def make_params(batch, num_heads, num_kv_heads, head_size, block_size, num_blocks,
                max_blocks_per_seq, causal, scale, block_table_stride=0,
                sliding_window=0, kv_cache_fp8=False, num_cus=0) -> AttnParams:
    """num_cus: compute units the planner fills (0: PA_PLAN_TARGET_CUS)."""
    return AttnParams(int(batch), int(num_heads), int(num_kv_heads), int(head_size),
                      int(block_size), int(num_blocks), int(max_blocks_per_seq),
                      int(block_table_stride), int(bool(causal)), float(np.float32(scale)),
                      int(sliding_window), int(bool(kv_cache_fp8)), int(num_cus))


def device_cus(device=None) -> int:
    """Compute units of a GPU, for AttnParams.num_cus."""
    import torch
    return int(torch.cuda.get_device_properties(device or torch.cuda.current_device())
               .multi_processor_count)


# --------------------------------------------------------------------------
# one-to-one wrappers
# --------------------------------------------------------------------------
def pa_plan_varlen(params: AttnParams, host_cu_seqlens_q, host_seqused_k,
                   force_splits: int = 0) -> Tuple[np.ndarray, PlanInfo]:
    """Host-only planner; returns (int32 work list, PlanInfo)."""
    cu = _i32(host_cu_seqlens_q)
    sk = _i32(host_seqused_k)
    info = PlanInfo()
    st = lib().pa_plan_varlen(ctypes.byref(params), _ptr_i32(cu), _ptr_i32(sk), int(force_splits),
                              None, 0, ctypes.byref(info))
    _check(st, "pa_plan_varlen(size)")
    wl = np.zeros(info.worklist_bytes // 4, dtype=np.int32)
    st = lib().pa_plan_varlen(ctypes.byref(params), _ptr_i32(cu), _ptr_i32(sk), int(force_splits),
                              _ptr_i32(wl), wl.nbytes, ctypes.byref(info))
    _check(st, "pa_plan_varlen")
    return wl, info


def pa_cascade_split(params: AttnParams, common_prefix_len: int, host_cu_seqlens_q,
                     host_seqused_k):
    """Host-only cascade metadata: (prefix_params, suffix_params, prefix_cu,
    prefix_seqused_k, suffix_seqused_k, block_table_col0)."""
    cu = _i32(host_cu_seqlens_q)
    sk = _i32(host_seqused_k)
    pp, sp = AttnParams(), AttnParams()
    pcu = np.zeros(2, np.int32)
    psk = np.zeros(1, np.int32)
    ssk = np.zeros(max(len(sk), 1), np.int32)
    col0 = np.zeros(1, np.int32)
    st = lib().pa_cascade_split(ctypes.byref(params), int(common_prefix_len), _ptr_i32(cu),
                                _ptr_i32(sk), ctypes.byref(pp), ctypes.byref(sp), _ptr_i32(pcu),
                                _ptr_i32(psk), _ptr_i32(ssk), _ptr_i32(col0))
    _check(st, "pa_cascade_split")
    return pp, sp, pcu, psk, ssk[:len(sk)], int(col0[0])


def pa_cascade_decide(params: AttnParams, host_cu_seqlens_q, host_seqused_k, host_block_table,
                      kv_bytes_per_elem: int = 2) -> Tuple[int, bool]:
    """Host-only cascade decision: (common_prefix_len, use_cascade)."""
    cu = _i32(host_cu_seqlens_q)
    sk = _i32(host_seqused_k)
    bt = _i32(host_block_table)
    P = np.zeros(1, np.int32)
    use = np.zeros(1, np.int32)
    st = lib().pa_cascade_decide(ctypes.byref(params), _ptr_i32(cu), _ptr_i32(sk), _ptr_i32(bt),
                                 int(kv_bytes_per_elem), _ptr_i32(P), _ptr_i32(use))
    _check(st, "pa_cascade_decide")
    return int(P[0]), bool(use[0])


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, what, dtype=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def pa_upload_words(host_words, device_words, stream=None):
    """Copy a pinned host int32 tensor into a device int32 tensor of the same
    size with a kernel on the stream (pa_upload_words).  The host tensor must
    stay unchanged until the copy has run."""
    import torch
    if not isinstance(host_words, torch.Tensor) or host_words.is_cuda or \
            not host_words.is_pinned():
        raise TypeError("host_words must be a pinned host tensor")
    if host_words.dtype != torch.int32 or not host_words.is_contiguous():
        raise TypeError("host_words must be contiguous int32")
    if device_words.numel() != host_words.numel() or not device_words.is_contiguous():
        raise ValueError("device_words must be a contiguous tensor of the same size")
    st = lib().pa_upload_words(ctypes.c_void_p(host_words.data_ptr()),
                               _dev(device_words, "device_words", torch.int32),
                               host_words.numel(), _stream(stream))
    _check(st, "pa_upload_words")


def pa_reshape_and_cache(key, value, kv_cache, slot_mapping, stream=None):
    """key/value: bf16 [T, Hkv, D] (row stride may exceed Hkv*D); kv_cache:
    bf16 [2, NB, BS, Hkv, D] contiguous; slot_mapping int64 [T]."""
    import torch
    T, Hkv, D = key.shape
    if value.shape != key.shape or key.stride(2) != 1 or value.stride(2) != 1 \
            or key.stride(1) != D or value.stride(1) != D:
        raise ValueError("key/value must be [T, Hkv, D] with contiguous heads")
    if not kv_cache.is_contiguous() or kv_cache.dim() != 5 or kv_cache.shape[0] != 2:
        raise ValueError("kv_cache must be a contiguous (2, NB, BS, Hkv, D) tensor")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    st = lib().pa_reshape_and_cache(
        _dev(key, "key", torch.bfloat16), _dev(value, "value", torch.bfloat16),
        key.stride(0), value.stride(0), _dev(kv_cache, "kv_cache", torch.bfloat16),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, Hkv, D, kv_cache.shape[1],
        kv_cache.shape[2], _stream(stream))
    _check(st, "pa_reshape_and_cache")


def _shape(t):
    return tuple(t.shape)


def check_fwd_args(params: AttnParams, plan: PlanInfo, worklist, q, kv_cache, cu_seqlens_q,
                   seqused_k, block_table, out, lse, fp8=False):
    """Host-side shape, stride and dtype checks of a forward call against its
    params and plan, before any launch: the kernels index these buffers with
    the shapes the params state, so a mismatch would read or write outside
    an allocation.  Raises ValueError."""
    T, H, D = int(plan.num_tokens), int(params.num_heads), int(params.head_size)
    B, Hkv = int(params.batch), int(params.num_kv_heads)
    for name, t in (("q", q), ("out", out)):
        if t is None or t.shape != (T, H, D) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{T}, {H}, {D}] tensor "
                             f"(plan.num_tokens, num_heads, head_size), got "
                             f"{None if t is None else _shape(t)}")
    if lse is not None and (lse.shape != (T, H) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous [{T}, {H}] tensor, got {_shape(lse)}")
    want_kv = (2, int(params.num_blocks), int(params.block_size), Hkv, D)
    if kv_cache.shape != want_kv or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache must be a contiguous {want_kv} tensor, got {_shape(kv_cache)}")
    if kv_cache.element_size() != (1 if fp8 else 2):
        raise ValueError("kv_cache element size does not match the cache format")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() < B + 1 or not cu_seqlens_q.is_contiguous():
        raise ValueError(f"cu_seqlens_q must be a contiguous int32 vector of {B + 1} entries")
    if seqused_k.dim() != 1 or seqused_k.numel() < B or not seqused_k.is_contiguous():
        raise ValueError(f"seqused_k must be a contiguous int32 vector of {B} entries")
    stride = int(params.block_table_stride) or int(params.max_blocks_per_seq)
    if B > 0 and (block_table.dim() != 2 or block_table.shape[0] < B
                  or block_table.shape[1] < params.max_blocks_per_seq
                  or block_table.stride(1) != 1
                  or (block_table.shape[0] > 1 and block_table.stride(0) != stride)):
        raise ValueError(f"block_table must be [>= {B}, >= {params.max_blocks_per_seq}] with row "
                         f"stride {stride}, got {_shape(block_table)} strides "
                         f"{tuple(block_table.stride())}")
    if worklist.numel() * worklist.element_size() < plan.worklist_bytes or \
            not worklist.is_contiguous():
        raise ValueError("worklist is smaller than plan.worklist_bytes")


def pa_varlen_fwd(params: AttnParams, plan: PlanInfo, worklist, q, kv_cache, cu_seqlens_q,
                  seqused_k, block_table, out, lse=None, workspace=None, stream=None):
    import torch
    check_fwd_args(params, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                   out, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_varlen_fwd(
        ctypes.byref(params), ctypes.byref(plan), _dev(worklist, "worklist", torch.int32),
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.bfloat16),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqused_k, "seqused_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), int(q.shape[0]),
        _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(st, "pa_varlen_fwd")


def pa_reshape_and_cache_fp8(key, value, kv_cache, slot_mapping, k_scale, v_scale, stream=None):
    """key/value: bf16 [T, Hkv, D]; kv_cache: uint8 (E4M3) [2, NB, BS, Hkv, D]
    contiguous; slot_mapping int64 [T]; k_scale/v_scale fp32 [Hkv]."""
    import torch
    T, Hkv, D = key.shape
    if value.shape != key.shape or key.stride(2) != 1 or value.stride(2) != 1 \
            or key.stride(1) != D or value.stride(1) != D:
        raise ValueError("key/value must be [T, Hkv, D] with contiguous heads")
    if not kv_cache.is_contiguous() or kv_cache.dim() != 5 or kv_cache.shape[0] != 2:
        raise ValueError("kv_cache must be a contiguous (2, NB, BS, Hkv, D) tensor")
    if slot_mapping.shape[0] != T or k_scale.numel() != Hkv or v_scale.numel() != Hkv:
        raise ValueError("slot_mapping must have one entry per token, the scales one per KV head")
    st = lib().pa_reshape_and_cache_fp8(
        _dev(key, "key", torch.bfloat16), _dev(value, "value", torch.bfloat16),
        key.stride(0), value.stride(0), _dev(kv_cache, "kv_cache", torch.uint8),
        _dev(slot_mapping, "slot_mapping", torch.int64), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), T, Hkv, D, kv_cache.shape[1], kv_cache.shape[2],
        _stream(stream))
    _check(st, "pa_reshape_and_cache_fp8")


def pa_varlen_fwd_fp8(params: AttnParams, plan: PlanInfo, worklist, q, kv_cache, cu_seqlens_q,
                      seqused_k, block_table, k_scale, v_scale, out, lse=None, workspace=None,
                      stream=None):
    import torch
    check_fwd_args(params, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                   out, lse, fp8=True)
    if k_scale.numel() != params.num_kv_heads or v_scale.numel() != params.num_kv_heads:
        raise ValueError("k_scale and v_scale need one entry per KV head")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_varlen_fwd_fp8(
        ctypes.byref(params), ctypes.byref(plan), _dev(worklist, "worklist", torch.int32),
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.uint8),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqused_k, "seqused_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), int(q.shape[0]),
        _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(st, "pa_varlen_fwd_fp8")


def pa_varlen_fwd_ex(params: AttnParams, plan: PlanInfo, worklist, q, kv_cache, cu_seqlens_q,
                     seqused_k, block_table, out, lse=None, workspace=None, stream=None,
                     k_scale=None, v_scale=None, s_aux=None):
    """bf16 cache, or (k_scale and v_scale given) a uint8 E4M3 cache;
    s_aux: None or fp32 [H] sink logits."""
    import torch
    fp8 = k_scale is not None or v_scale is not None
    check_fwd_args(params, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                   out, lse, fp8=fp8)
    if fp8 and (k_scale is None or v_scale is None or k_scale.numel() != params.num_kv_heads
                or v_scale.numel() != params.num_kv_heads):
        raise ValueError("k_scale and v_scale need one entry per KV head")
    if s_aux is not None and s_aux.numel() != params.num_heads:
        raise ValueError("s_aux needs one entry per query head")
    opt = FwdOptions(PA_KV_E4M3 if fp8 else PA_KV_BF16,
                     _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
                     _dev(s_aux, "s_aux", torch.float32))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_varlen_fwd_ex(
        ctypes.byref(params), ctypes.byref(plan), _dev(worklist, "worklist", torch.int32),
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.uint8 if fp8 else torch.bfloat16),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqused_k, "seqused_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), ctypes.byref(opt), int(q.shape[0]),
        _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(st, "pa_varlen_fwd_ex")


def pa_varlen_fwd_noalloc(params: AttnParams, plan: PlanInfo, worklist, q, kv_cache, cu_seqlens_q,
                          seqused_k, block_table, out, lse=None, stream=None, k_scale=None,
                          v_scale=None, s_aux=None):
    """pa_varlen_fwd_ex without a workspace: the partials go to the library's
    own device scratch (PA_NOALLOC_SCRATCH_BYTES per GPU)."""
    import torch
    fp8 = k_scale is not None or v_scale is not None
    check_fwd_args(params, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                   out, lse, fp8=fp8)
    if fp8 and (k_scale is None or v_scale is None or k_scale.numel() != params.num_kv_heads
                or v_scale.numel() != params.num_kv_heads):
        raise ValueError("k_scale and v_scale need one entry per KV head")
    if s_aux is not None and s_aux.numel() != params.num_heads:
        raise ValueError("s_aux needs one entry per query head")
    opt = FwdOptions(PA_KV_E4M3 if fp8 else PA_KV_BF16,
                     _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
                     _dev(s_aux, "s_aux", torch.float32))
    st = lib().pa_varlen_fwd_noalloc(
        ctypes.byref(params), ctypes.byref(plan), _dev(worklist, "worklist", torch.int32),
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.uint8 if fp8 else torch.bfloat16),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqused_k, "seqused_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), ctypes.byref(opt), int(q.shape[0]),
        _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32), _stream(stream))
    _check(st, "pa_varlen_fwd_noalloc")


def pa_merge_attn_states(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse,
                         stream=None):
    import torch
    T, H, D = prefix_out.shape
    for t in (out, prefix_out, suffix_out):
        if not t.is_contiguous() or tuple(t.shape) != (T, H, D):
            raise ValueError("merge operands must be contiguous [T, H, D]")
    for t in (prefix_lse, suffix_lse) + ((out_lse,) if out_lse is not None else ()):
        if not t.is_contiguous() or tuple(t.shape) != (T, H):
            raise ValueError("lse operands must be contiguous [T, H]")
    st = lib().pa_merge_attn_states(
        _dev(out, "out", torch.bfloat16), _dev(out_lse, "out_lse", torch.float32),
        _dev(prefix_out, "prefix_out", torch.bfloat16), _dev(prefix_lse, "prefix_lse", torch.float32),
        _dev(suffix_out, "suffix_out", torch.bfloat16), _dev(suffix_lse, "suffix_lse", torch.float32),
        T, H, D, _stream(stream))
    _check(st, "pa_merge_attn_states")


# --------------------------------------------------------------------------
# conveniences
# --------------------------------------------------------------------------
class VarlenPlan:
    """A planned call: params, host + device work list, device workspace."""

    def __init__(self, params: AttnParams, host_cu_seqlens_q, host_seqused_k,
                 force_splits: int = 0, device=None):
        import torch
        self.params = params
        self.host_worklist, self.info = pa_plan_varlen(params, host_cu_seqlens_q, host_seqused_k,
                                                       force_splits)
        device = device or torch.device("cuda")
        self.worklist = torch.from_numpy(self.host_worklist).to(device)
        nbytes = max(int(self.info.workspace_bytes), 0)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def plan_varlen(q_shape, kv_cache_shape, block_table_shape, host_cu_seqlens_q, host_seqused_k,
                scale, causal, force_splits=0, block_table_stride=0,
                sliding_window=0, kv_cache_fp8=False) -> VarlenPlan:
    T, H, D = q_shape
    _, NB, BS, Hkv, D2 = kv_cache_shape
    if D2 != D:
        raise ValueError("head size of q and kv_cache differ")
    B, MB = block_table_shape
    p = make_params(B, H, Hkv, D, BS, NB, MB, causal, scale, block_table_stride, sliding_window,
                    kv_cache_fp8, num_cus=device_cus())
    return VarlenPlan(p, host_cu_seqlens_q, host_seqused_k, force_splits)


def varlen_fwd(q, kv_cache, cu_seqlens_q, seqused_k, block_table, plan: VarlenPlan,
               out=None, lse=None, stream=None, k_scale=None, v_scale=None, s_aux=None):
    """bf16 cache, or (k_scale and v_scale given) a uint8 E4M3 cache;
    s_aux: optional fp32 [H] sink logits."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    if s_aux is not None:
        pa_varlen_fwd_ex(plan.params, plan.info, plan.worklist, q, kv_cache, cu_seqlens_q,
                         seqused_k, block_table, out, lse, plan.workspace, stream,
                         k_scale, v_scale, s_aux)
    elif k_scale is None and v_scale is None:
        pa_varlen_fwd(plan.params, plan.info, plan.worklist, q, kv_cache, cu_seqlens_q, seqused_k,
                      block_table, out, lse, plan.workspace, stream)
    else:
        pa_varlen_fwd_fp8(plan.params, plan.info, plan.worklist, q, kv_cache, cu_seqlens_q,
                          seqused_k, block_table, k_scale, v_scale, out, lse, plan.workspace,
                          stream)
    return out, lse


class CascadePlan:
    """Both cascade passes planned, with their small device metadata."""

    def __init__(self, q_shape, kv_cache_shape, block_table_shape, host_cu_seqlens_q,
                 host_seqused_k, scale, common_prefix_len, force_splits=0):
        import torch
        T, H, D = q_shape
        _, NB, BS, Hkv, _ = kv_cache_shape
        B, MB = block_table_shape
        full = make_params(B, H, Hkv, D, BS, NB, MB, True, scale, num_cus=device_cus())
        pp, sp, pcu, psk, ssk, col0 = pa_cascade_split(full, common_prefix_len,
                                                       host_cu_seqlens_q, host_seqused_k)
        self.prefix = VarlenPlan(pp, pcu, psk, force_splits)
        self.suffix = VarlenPlan(sp, host_cu_seqlens_q, ssk, force_splits)
        dev = torch.device("cuda")
        self.prefix_cu = torch.from_numpy(pcu).to(dev)
        self.prefix_seqused_k = torch.from_numpy(psk).to(dev)
        self.suffix_seqused_k = torch.from_numpy(ssk).to(dev)
        self.col0 = col0


def cascade_fwd(q, kv_cache, cu_seqlens_q, block_table, plan: CascadePlan, out=None, lse=None,
                prefix_out=None, prefix_lse=None, suffix_out=None, suffix_lse=None, stream=None):
    """Prefix pass + suffix pass + merge.  Returns (out, lse)."""
    import torch
    T, H, D = q.shape
    dev = q.device
    if prefix_out is None:
        prefix_out = torch.empty_like(q)
        suffix_out = torch.empty_like(q)
        prefix_lse = torch.empty(T, H, dtype=torch.float32, device=dev)
        suffix_lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous")
    pa_varlen_fwd(plan.prefix.params, plan.prefix.info, plan.prefix.worklist, q, kv_cache,
                  plan.prefix_cu, plan.prefix_seqused_k, block_table, prefix_out, prefix_lse,
                  plan.prefix.workspace, stream)
    suffix_bt = block_table[:, plan.col0:]   # strided view: same row stride
    pa_varlen_fwd(plan.suffix.params, plan.suffix.info, plan.suffix.worklist, q, kv_cache,
                  cu_seqlens_q, plan.suffix_seqused_k, suffix_bt, suffix_out, suffix_lse,
                  plan.suffix.workspace, stream)
    pa_merge_attn_states(out, lse, prefix_out, prefix_lse, suffix_out, suffix_lse, stream)
    return out, lse
