"""Thin ctypes binding of libcb.so (include/cb.h and its optional extensions include/cb_ext.h).
Argument marshalling only.

Every function here has the name of the C entry point it calls and forwards to it: torch tensors
become raw pointers (host or device), the HIP stream defaults to torch's current stream on the
tensor's device, and a non-zero status becomes a ``CbError``.  No part of the step is computed in
Python: scheduling runs in the C++ builder and all device work in the library's HIP kernels.
Loading fails loudly when libcb.so has not been built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; CB_LIBCB_PATH names another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("CB_LIBCB_PATH") or os.path.join(_PKG, "libcb.so")

CB_OK, CB_ERR_INVALID, CB_ERR_DECODE_OVER_BUDGET, CB_ERR_OUT_OF_BLOCKS, CB_ERR_CAPACITY, CB_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
CB_F32, CB_BF16 = 0, 1
CB_POLICY_DECODE_FIRST, CB_POLICY_PREFILL_FIRST, CB_POLICY_FAIR_SHARE = 0, 1, 2

_i32, _i64, _sz, _vp, _f32, _f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_float, ctypes.c_double)
_pi32 = ctypes.POINTER(ctypes.c_int32)


class CbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().cb_status_string(status).decode()} (status {status})")


class cb_sched_config(ctypes.Structure):
    _fields_ = [("block_size", _i32), ("num_blocks", _i32), ("free_list", _pi32), ("max_chunk", _i32),
                ("prefill_floor", _i32), ("max_partial_prefills", _i32), ("max_num_seqs", _i32),
                ("policy", _i32), ("decode_share_pct", _i32), ("prefill_quota_pct", _i32)]


class cb_step(ctypes.Structure):
    _fields_ = [("cap_seqs", _i32), ("cap_tokens", _i32), ("cap_blocks", _i32),
                ("seq_ids", _pi32), ("cu_seqlens_q", _pi32), ("context_lens", _pi32),
                ("cu_blocks", _pi32), ("block_table", _pi32), ("positions", _pi32),
                ("slot_mapping", _pi32),
                ("num_seqs", _i32), ("num_decodes", _i32), ("num_tokens", _i32),
                ("num_prefill_tokens", _i32), ("unused_tokens", _i32), ("max_q_len", _i32),
                ("max_context_len", _i32), ("max_decode_context_len", _i32),
                ("num_blocks_emitted", _i32)]


_LIB = None

EXPORTS = {
    "cb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cb_sched_create": (ctypes.c_int, [ctypes.POINTER(cb_sched_config), ctypes.POINTER(_vp)]),
    "cb_sched_destroy": (None, [_vp]),
    "cb_sched_clone": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
    "cb_sched_add_running": (ctypes.c_int, [_vp, _i32, _pi32]),
    "cb_sched_add_prompt": (ctypes.c_int, [_vp, _i32, _i32, _pi32]),
    "cb_sched_get_blocks": (ctypes.c_int, [_vp, _i32, _pi32, _i32, _pi32]),
    "cb_sched_finish": (ctypes.c_int, [_vp, _i32]),
    "cb_linear_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "cb_linear": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz]),
    "cb_sched_pending_prompts": (ctypes.c_int, [_vp, _pi32]),
    "cb_sched_free_blocks": (ctypes.c_int, [_vp, _pi32]),
    "cb_build_step": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(cb_step)]),
    "cb_copy_host_to_device": (ctypes.c_int, [_vp, _vp, _vp, _sz]),
    "cb_rope_cos_sin": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), _i32, _i32, _f64]),
    "cb_rope_kv_append": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64]),
    "cb_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "cb_mixed_paged_attention": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp,
                                                _vp, _vp, _vp, _vp, _vp, _sz]),
    "cb_mixed_paged_attention_noalloc": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                        _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                                        _vp, _vp, _vp, _vp, _vp]),
    "cb_mixed_paged_attention_timed": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _sz, _vp, _i32, ctypes.POINTER(_vp)]),
    "cb_attn_decode_waves": (_i32, [_vp, _i32]),
    "cb_decode_plan_ints": (_sz, [_i32, _i32]),
    "cb_decode_plan": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32, _pi32, _sz]),
}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m chunked_prefill_mixed_decode_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int, where: str):
    if status != CB_OK:
        raise CbError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _i32ptr(t):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), _pi32)


def _stream(t, stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return CB_F32
    if dt == torch.bfloat16:
        return CB_BF16
    raise ValueError(f"unsupported element type {dt}")


# ---- host builder ------------------------------------------------------------------------------

class Sched:
    """Owner of one ``cb_sched`` (freed with the object)."""

    def __init__(self, handle):
        self.handle = handle

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.cb_sched_destroy(self.handle)
            self.handle = None


def cb_sched_create(block_size: int, num_blocks: int, free_list=None, max_chunk: int = 0,
                    prefill_floor: int = 0, max_partial_prefills: int = 0, max_num_seqs: int = 0,
                    policy: int = CB_POLICY_DECODE_FIRST, decode_share_pct: int = 0,
                    prefill_quota_pct: int = 0) -> Sched:
    cfg = cb_sched_config(block_size, num_blocks, None, max_chunk, prefill_floor,
                          max_partial_prefills, max_num_seqs, policy, decode_share_pct,
                          prefill_quota_pct)
    keep = None
    if free_list is not None:
        keep = (ctypes.c_int32 * len(free_list))(*free_list)
        cfg.free_list = ctypes.cast(keep, _pi32)
    h = _vp()
    _check(_lib().cb_sched_create(ctypes.byref(cfg), ctypes.byref(h)), "cb_sched_create")
    return Sched(h)


def cb_sched_clone(s: Sched) -> Sched:
    h = _vp()
    _check(_lib().cb_sched_clone(s.handle, ctypes.byref(h)), "cb_sched_clone")
    return Sched(h)


def cb_sched_add_running(s: Sched, context_len: int) -> int:
    rid = ctypes.c_int32()
    _check(_lib().cb_sched_add_running(s.handle, context_len, ctypes.byref(rid)), "cb_sched_add_running")
    return rid.value


def cb_sched_add_prompt(s: Sched, prompt_len: int, cached_len: int = 0) -> int:
    rid = ctypes.c_int32()
    _check(_lib().cb_sched_add_prompt(s.handle, prompt_len, cached_len, ctypes.byref(rid)),
           "cb_sched_add_prompt")
    return rid.value


def cb_sched_get_blocks(s: Sched, req_id: int) -> list[int]:
    n = ctypes.c_int32()
    st = _lib().cb_sched_get_blocks(s.handle, req_id, None, 0, ctypes.byref(n))
    if st not in (CB_OK, CB_ERR_CAPACITY):
        _check(st, "cb_sched_get_blocks")
    buf = (ctypes.c_int32 * max(n.value, 1))()
    _check(_lib().cb_sched_get_blocks(s.handle, req_id, buf, n.value, ctypes.byref(n)), "cb_sched_get_blocks")
    return list(buf[:n.value])


def cb_sched_pending_prompts(s: Sched) -> int:
    n = ctypes.c_int32()
    _check(_lib().cb_sched_pending_prompts(s.handle, ctypes.byref(n)), "cb_sched_pending_prompts")
    return n.value


def cb_sched_free_blocks(s: Sched) -> int:
    n = ctypes.c_int32()
    _check(_lib().cb_sched_free_blocks(s.handle, ctypes.byref(n)), "cb_sched_free_blocks")
    return n.value


def cb_sched_finish(s: Sched, req_id: int) -> None:
    _check(_lib().cb_sched_finish(s.handle, req_id), "cb_sched_finish")


STEP_ARRAYS = ("seq_ids", "cu_seqlens_q", "context_lens", "cu_blocks", "block_table",
               "positions", "slot_mapping")
STEP_SCALARS = ("num_seqs", "num_decodes", "num_tokens", "num_prefill_tokens", "unused_tokens",
                "max_q_len", "max_context_len", "max_decode_context_len", "num_blocks_emitted")


class StepBuffers:
    """Host int32 arrays that cb_build_step fills, packed in one flat buffer (pinned when a GPU is
    present) so that a step's metadata reaches the device in a single asynchronous copy."""

    def __init__(self, cap_seqs: int, cap_tokens: int, cap_blocks: int, pin: bool | None = None,
                 plan_ints: int = 0):
        if pin is None:
            pin = torch.cuda.is_available()
        self.cap = (cap_seqs, cap_tokens, cap_blocks)
        sizes = {"seq_ids": cap_seqs, "cu_seqlens_q": cap_seqs + 1, "context_lens": cap_seqs,
                 "cu_blocks": cap_seqs + 1, "block_table": max(cap_blocks, 1),
                 "positions": max(cap_tokens, 1), "slot_mapping": max(cap_tokens, 1)}
        names = STEP_ARRAYS
        if plan_ints:                                  # a host-made decode plan travels along
            sizes["decode_plan"] = plan_ints
            names = STEP_ARRAYS + ("decode_plan",)
        self.offsets = {}
        off = 0
        for k in names:
            self.offsets[k] = off
            off += (sizes[k] + 63) // 64 * 64          # 256-byte aligned sub-arrays
        self.flat = torch.zeros(off, dtype=torch.int32, pin_memory=pin)
        self.arrays = {k: self.flat[self.offsets[k]:self.offsets[k] + sizes[k]] for k in names}
        self.step = cb_step()
        for k in STEP_ARRAYS:
            setattr(self.step, k, _i32ptr(self.arrays[k]))


@dataclasses.dataclass
class StepMeta:
    """Scalars of a built step plus views of its host arrays (valid until the next build)."""
    num_seqs: int
    num_decodes: int
    num_tokens: int
    num_prefill_tokens: int
    unused_tokens: int
    max_q_len: int
    max_context_len: int
    max_decode_context_len: int
    num_blocks_emitted: int
    host: dict

    def lengths(self) -> dict:
        return {"seq_ids": self.num_seqs, "cu_seqlens_q": self.num_seqs + 1,
                "context_lens": self.num_seqs, "cu_blocks": self.num_seqs + 1,
                "block_table": self.num_blocks_emitted, "positions": self.num_tokens,
                "slot_mapping": self.num_tokens}


def cb_build_step(s: Sched, token_budget: int, buf: StepBuffers) -> StepMeta:
    st = buf.step
    st.cap_seqs, st.cap_tokens, st.cap_blocks = buf.cap
    _check(_lib().cb_build_step(s.handle, token_budget, ctypes.byref(st)), "cb_build_step")
    scal = {k: getattr(st, k) for k in STEP_SCALARS}
    meta = StepMeta(**scal, host={})
    meta.host = {k: buf.arrays[k][:n] for k, n in meta.lengths().items()}
    meta.launch_tokens = meta.num_tokens            # rows the step's launches cover (padding: more)
    return meta


# ---- rotary table (host) ------------------------------------------------------------------------

def cb_rope_cos_sin(max_pos: int, D: int, base: float = 10000.0) -> torch.Tensor:
    out = torch.empty((max_pos, D), dtype=torch.float32)
    _check(_lib().cb_rope_cos_sin(ctypes.cast(ctypes.c_void_p(out.data_ptr()), ctypes.POINTER(ctypes.c_float)),
                                  max_pos, D, base), "cb_rope_cos_sin")
    return out


# ---- device ops ----------------------------------------------------------------------------------

def cb_copy_host_to_device(src, dst, stream=None):
    """src: pinned host tensor; dst: device tensor of at least as many bytes (kernel copy on the
    stream, no copy engine)."""
    nbytes = src.numel() * src.element_size()
    if not src.is_pinned() or dst.numel() * dst.element_size() < nbytes:
        raise ValueError("cb_copy_host_to_device: src must be pinned and dst large enough")
    _check(_lib().cb_copy_host_to_device(_stream(dst, stream), _ptr(src), _ptr(dst), nbytes),
           "cb_copy_host_to_device")


def cb_rope_kv_append(q, k, v, positions, slot_mapping, cos_sin, q_out, k_cache, v_cache,
                      stream=None):
    """q, q_out [T, Hq, D] (q may be None); k, v [T, Hkv, D]; caches [nb, Hkv, bs, D]."""
    T, Hkv, D = k.shape
    Hq = q.shape[1] if q is not None else 0
    nb, _, bs, _ = k_cache.shape
    _check(_lib().cb_rope_kv_append(
        _stream(k, stream), dtype_code(k.dtype), T, max(Hq, 1), Hkv, D, bs, _ptr(q), _ptr(k), _ptr(v),
        _ptr(positions), _ptr(slot_mapping), _ptr(cos_sin), cos_sin.shape[0], _ptr(q_out),
        _ptr(k_cache), _ptr(v_cache), nb), "cb_rope_kv_append")


def cb_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib().cb_linear_workspace_bytes(M, N, K))


def cb_linear(x, w, y, workspace=None, stream=None):
    """y [M, N] = x [M, K] . w [N, K]^T (bfloat16 device tensors, contiguous); ``workspace`` a device
    tensor of at least cb_linear_workspace_bytes(M, N, K) bytes when that is not 0."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("cb_linear: shapes do not match")
    for t in (x, w, y):
        if not t.is_contiguous():
            raise ValueError("cb_linear: tensors must be contiguous")
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib().cb_linear(_stream(x, stream), dtype_code(x.dtype), M, N, K, _ptr(x), _ptr(w), _ptr(y),
                            _ptr(workspace), nbytes), "cb_linear")


def cb_attn_workspace_bytes(num_seqs, num_decodes, T, max_q_len, max_decode_ctx, max_ctx, Hq, Hkv, D) -> int:
    return int(_lib().cb_attn_workspace_bytes(num_seqs, num_decodes, T, max_q_len, max_decode_ctx,
                                              max_ctx, Hq, Hkv, D))


def _stream_arg(device_or_stream) -> int:
    """hipStream_t of a torch stream, or the current stream of a device (None: the current one).
    Without a usable GPU: the null stream (the library then assumes MI355X's 256 compute units)."""
    st = device_or_stream
    if isinstance(st, torch.cuda.Stream):
        return st.cuda_stream
    if st is None or isinstance(st, (torch.device, int, str)):
        return torch.cuda.current_stream(st).cuda_stream if torch.cuda.is_available() else 0
    return int(st)


def cb_attn_decode_waves(device_or_stream=None, has_chunks: bool = True) -> int:
    """Decode waves an attention call launches on the device of the stream (default: current)."""
    return int(_lib().cb_attn_decode_waves(ctypes.c_void_p(_stream_arg(device_or_stream)),
                                           int(bool(has_chunks))))


def cb_decode_plan_ints(num_decodes: int, n_waves: int) -> int:
    return int(_lib().cb_decode_plan_ints(num_decodes, n_waves))


def cb_decode_plan(cu_seqlens_q, context_lens, num_decodes: int, max_q_len: int, max_ctx: int,
                   Hq: int, Hkv: int, out, device_or_stream=None) -> int:
    """Host-made decode split for an attention call over the step (num_seqs = len(context_lens)
    rows, decode rows first) with the same shape arguments.  cu_seqlens_q, context_lens: host int32
    tensors (cu_seqlens_q may be None when every row decodes); out: host int32 tensor of at least
    cb_decode_plan_ints(num_decodes, n_waves) entries.  The plan is for an attention call on the
    device of the stream (default: current); returns its wave count (the call's plan_waves)."""
    tensors = [t for t in (cu_seqlens_q, context_lens, out) if t is not None]
    if any(t.dtype != torch.int32 or t.is_cuda for t in tensors):
        raise ValueError("cb_decode_plan: int32 host tensors")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("cb_decode_plan: contiguous tensors")
    num_seqs = context_lens.numel()
    if cu_seqlens_q is not None and cu_seqlens_q.numel() < num_seqs + 1:
        raise ValueError("cb_decode_plan: cu_seqlens_q needs num_seqs + 1 entries")
    _check(_lib().cb_decode_plan(ctypes.c_void_p(_stream_arg(device_or_stream)), num_seqs, num_decodes,
                                 max_q_len, max_ctx, Hq, Hkv,
                                 _i32ptr(cu_seqlens_q) if cu_seqlens_q is not None else None,
                                 _i32ptr(context_lens), _i32ptr(out), out.numel()), "cb_decode_plan")
    return int(out[3])


def cb_mixed_paged_attention(q, k_cache, v_cache, cu_seqlens_q, context_lens, cu_blocks,
                             block_table, out, workspace, *, num_seqs, num_decodes, max_q_len,
                             max_decode_ctx, max_ctx, scale, stream=None, events=None,
                             decode_plan=None, plan_waves: int = 0):
    """q, out [T, Hq, D]; caches [nb, Hkv, bs, D]; int32 metadata on the device; decode_plan: the
    device copy of a cb_decode_plan output (or None: the split runs on the device)."""
    T, Hq, D = q.shape
    _, Hkv, bs, _ = k_cache.shape
    args = (_stream(q, stream), dtype_code(q.dtype), num_seqs, num_decodes, T, max_q_len,
            max_decode_ctx, max_ctx, Hq, Hkv, D, bs, scale, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(cu_seqlens_q), _ptr(context_lens), _ptr(cu_blocks), _ptr(block_table), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size() if workspace is not None else 0)
    if events is None and decode_plan is None:
        _check(_lib().cb_mixed_paged_attention(*args), "cb_mixed_paged_attention")
    else:
        ev = None
        if events is not None:
            if len(events) != 6:
                raise ValueError("events: six torch.cuda.Event (or None) entries")
            ev = (_vp * 6)(*[ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events])
        _check(_lib().cb_mixed_paged_attention_timed(*args, _ptr(decode_plan), plan_waves, ev),
               "cb_mixed_paged_attention_timed")


def cb_mixed_paged_attention_noalloc(q, k_cache, v_cache, cu_seqlens_q, context_lens, cu_blocks,
                                     block_table, out, *, num_seqs, num_decodes, max_q_len,
                                     max_decode_ctx, max_ctx, scale, stream=None):
    """cb_mixed_paged_attention without a workspace (the library's per-GPU scratch array)."""
    T, Hq, D = q.shape
    _, Hkv, bs, _ = k_cache.shape
    _check(_lib().cb_mixed_paged_attention_noalloc(
        _stream(q, stream), dtype_code(q.dtype), num_seqs, num_decodes, T, max_q_len, max_decode_ctx,
        max_ctx, Hq, Hkv, D, bs, scale, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
        _ptr(context_lens), _ptr(cu_blocks), _ptr(block_table), _ptr(out)), "cb_mixed_paged_attention_noalloc")
