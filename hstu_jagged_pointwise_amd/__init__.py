"""MI355X (gfx950) HSTU jagged attention: thin Python binding over the C ABI in include/hstu.h.

Every function here only marshals arguments (torch device tensors -> raw pointers, the current
HIP stream) and calls the function of the same name in ``_build/libhstu_amd.so``.  All arithmetic
runs in the library's HIP kernels; there is no fallback: if the library is not built, or the
tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libhstu_amd.so")

HSTU_F32 = 0
HSTU_BF16 = 1
HSTU_PLAN_HOST_ONLY = 1
OP_FWD, OP_FWD_GATED, OP_BWD, OP_LAYER, OP_LAYER_BWD, OP_CACHED = 0, 1, 2, 3, 4, 5


class HstuAttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("max_seqlen", ctypes.c_int32),
        ("num_contexts", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("qkv_token_stride", ctypes.c_int64),
        ("timestamps", ctypes.c_void_p),
        ("rab_pos", ctypes.c_void_p),
        ("rab_ts", ctypes.c_void_p),
    ]


class HstuPlanInfo(ctypes.Structure):
    _fields_ = [
        ("visible_pairs", ctypes.c_int64),
        ("fwd_units", ctypes.c_int64),
        ("bwd_units", ctypes.c_int64),
        ("fwd_tiles", ctypes.c_int64),
        ("fwd_row_block", ctypes.c_int64),
        ("bwd_key_block", ctypes.c_int64),
        ("fwd_items", ctypes.c_int64),
        ("fwd_split_blocks", ctypes.c_int64),
        ("bwd_stored_ds", ctypes.c_int64),
        ("bwd_ds_bytes", ctypes.c_int64),
        ("fwd_item_rows", ctypes.c_int64),
    ]


EXPORTS = ["hstu_status_str", "hstu_plan_create", "hstu_plan_destroy", "hstu_plan_destroy_on",
           "hstu_plan_info",
           "hstu_plan_units", "hstu_workspace_bytes", "hstu_attn_fwd", "hstu_attn_fwd_noalloc",
           "hstu_attn_bwd",
           "hstu_attn_bwd_dkdv", "hstu_attn_bwd_dq", "hstu_layer_fwd", "hstu_layer_bwd",
           "hstu_plan_create_cached", "hstu_attn_fwd_cached", "hstu_jagged_select"]

_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library missing: {path} (build it with __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    argp = ctypes.POINTER(HstuAttnArgs)
    lib.hstu_status_str.argtypes = [I32]
    lib.hstu_status_str.restype = ctypes.c_char_p
    lib.hstu_plan_create.argtypes = [argp, P, P, U32, ctypes.POINTER(P)]
    lib.hstu_plan_create.restype = I32
    lib.hstu_plan_destroy.argtypes = [P]
    lib.hstu_plan_destroy.restype = None
    lib.hstu_plan_destroy_on.argtypes = [P, P]
    lib.hstu_plan_destroy_on.restype = None
    lib.hstu_plan_info.argtypes = [P, ctypes.POINTER(HstuPlanInfo)]
    lib.hstu_plan_info.restype = I32
    lib.hstu_plan_units.argtypes = [P, I32, P, I64, ctypes.POINTER(I64)]
    lib.hstu_plan_units.restype = I32
    lib.hstu_workspace_bytes.argtypes = [P, I32, I32]
    lib.hstu_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_attn_fwd.argtypes = [P, argp, P, P, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.hstu_attn_fwd.restype = I32
    lib.hstu_attn_fwd_noalloc.argtypes = [P, argp, P, P, P, P, ctypes.c_float, P, P]
    lib.hstu_attn_fwd_noalloc.restype = I32
    lib.hstu_attn_bwd.argtypes = [P, argp, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hstu_attn_bwd.restype = I32
    lib.hstu_attn_bwd_dkdv.argtypes = [P, argp, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hstu_attn_bwd_dkdv.restype = I32
    lib.hstu_attn_bwd_dq.argtypes = [P, argp, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hstu_attn_bwd_dq.restype = I32
    lib.hstu_layer_fwd.argtypes = [P, argp, I32, P, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.hstu_layer_fwd.restype = I32
    lib.hstu_layer_bwd.argtypes = [P, argp, I32, P, P, P, P, ctypes.c_float, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
    lib.hstu_layer_bwd.restype = I32
    lib.hstu_plan_create_cached.argtypes = [argp, P, P, U32, ctypes.POINTER(P)]
    lib.hstu_plan_create_cached.restype = I32
    lib.hstu_attn_fwd_cached.argtypes = [P, argp, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hstu_attn_fwd_cached.restype = I32
    lib.hstu_jagged_select.argtypes = [I32, P, I64, P, I64, P, I64, P, P, P]
    lib.hstu_jagged_select.restype = I32
    _lib = lib
    return lib


class HstuError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(f"hstu status {self.status}: {hstu_status_str(self.status)}")


def _check(status: int) -> None:
    if status != 0:
        raise HstuError(status)


def hstu_status_str(status: int) -> str:
    return load_library().hstu_status_str(int(status)).decode()


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def make_args(*, dtype: int, batch: int, num_heads: int, head_dim: int, total_tokens: int,
              max_seqlen: int, num_contexts: int = 0, alpha: float = 1.0,
              qkv_token_stride: int = 0, timestamps=None, rab_pos=None, rab_ts=None) -> HstuAttnArgs:
    """Fill the C argument struct; tensor arguments are torch device tensors or None."""
    return HstuAttnArgs(int(dtype), int(batch), int(num_heads), int(head_dim), int(total_tokens),
                        int(max_seqlen), int(num_contexts), float(alpha), 0,
                        int(qkv_token_stride),
                        None if timestamps is None else _ptr(timestamps),
                        None if rab_pos is None else _ptr(rab_pos),
                        None if rab_ts is None else _ptr(rab_ts))


class Plan:
    """Owns a hstu_plan_t*.  close() (or garbage collection) frees it with hstu_plan_destroy, which
    waits for the device; close(stream) frees it in the order of that stream instead
    (hstu_plan_destroy_on), after the calls already queued there."""

    def __init__(self, handle: int, args: HstuAttnArgs):
        self.handle = handle
        self.args = args

    def close(self, stream=None) -> None:
        if self.handle:
            lib = load_library()
            if stream is None:
                lib.hstu_plan_destroy(ctypes.c_void_p(self.handle))
            else:
                lib.hstu_plan_destroy_on(ctypes.c_void_p(self.handle), _stream(stream))
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def hstu_plan_create(args: HstuAttnArgs, seq_offsets, num_targets=None, flags: int = 0) -> Plan:
    """seq_offsets / num_targets are host arrays (numpy or CPU tensors)."""
    off = np.ascontiguousarray(np.asarray(seq_offsets), dtype=np.int64)
    nt = None if num_targets is None else np.ascontiguousarray(np.asarray(num_targets), dtype=np.int32)
    handle = ctypes.c_void_p()
    _check(load_library().hstu_plan_create(
        ctypes.byref(args), off.ctypes.data_as(ctypes.c_void_p),
        None if nt is None else nt.ctypes.data_as(ctypes.c_void_p), int(flags),
        ctypes.byref(handle)))
    return Plan(handle.value, args)


def hstu_plan_create_cached(args: HstuAttnArgs, cand_offsets, cache_offsets,
                            flags: int = 0) -> Plan:
    """Plan for candidate scoring against cached history; offsets are host arrays."""
    co = np.ascontiguousarray(np.asarray(cand_offsets), dtype=np.int64)
    ho = np.ascontiguousarray(np.asarray(cache_offsets), dtype=np.int64)
    handle = ctypes.c_void_p()
    _check(load_library().hstu_plan_create_cached(
        ctypes.byref(args), co.ctypes.data_as(ctypes.c_void_p),
        ho.ctypes.data_as(ctypes.c_void_p), int(flags), ctypes.byref(handle)))
    return Plan(handle.value, args)


def hstu_plan_destroy(plan: Plan) -> None:
    plan.close()


def hstu_plan_destroy_on(plan: Plan, stream=None) -> None:
    """Frees the plan in the order of `stream` (torch's current stream when None)."""
    plan.close(torch_current_stream() if stream is None else stream)


def torch_current_stream():
    import torch
    return torch.cuda.current_stream()


def hstu_plan_info(plan: Plan) -> dict:
    info = HstuPlanInfo()
    _check(load_library().hstu_plan_info(ctypes.c_void_p(plan.handle), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in HstuPlanInfo._fields_}


def hstu_plan_units(plan: Plan, op: int) -> np.ndarray:
    """op 0 / 1 / 3: (count, 4) work units; op 2: (count, 8) bf16 forward items."""
    lib = load_library()
    count = ctypes.c_int64()
    _check(lib.hstu_plan_units(ctypes.c_void_p(plan.handle), int(op), None, 0, ctypes.byref(count)))
    out = np.zeros((count.value, 8 if op == 2 else 4), np.int32)
    _check(lib.hstu_plan_units(ctypes.c_void_p(plan.handle), int(op),
                               out.ctypes.data_as(ctypes.c_void_p), count.value,
                               ctypes.byref(count)))
    return out


def hstu_workspace_bytes(plan: Plan, op: int, d_model: int = 0) -> int:
    return int(load_library().hstu_workspace_bytes(ctypes.c_void_p(plan.handle), int(op),
                                                   int(d_model)))


def _workspace(plan: Plan, op: int, d_model: int, ws, device, stream=None):
    """The caller's workspace, or a temporary one from torch's allocator.  A temporary is
    allocated on torch's current stream; when the call is queued on another stream it is marked
    as used there, so torch does not hand the memory out again before that stream's work ends."""
    need = hstu_workspace_bytes(plan, op, d_model)
    if ws is None and need > 0:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(_torch_stream(stream, device))
    return ws, (ws.numel() * ws.element_size() if ws is not None else 0)


def _torch_stream(stream, device):
    import torch
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def hstu_attn_fwd(plan: Plan, args: HstuAttnArgs, q, k, v, out, u=None, ln_eps: float = 1e-5,
                  ws=None, stream=None) -> None:
    ws, nbytes = _workspace(plan, OP_FWD_GATED if u is not None else OP_FWD, 0, ws, q.device, stream)
    _check(load_library().hstu_attn_fwd(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(u),
        float(ln_eps), _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def hstu_attn_fwd_noalloc(plan: Plan, args: HstuAttnArgs, q, k, v, out, u=None,
                          ln_eps: float = 1e-5, stream=None) -> None:
    """hstu_attn_fwd with its scratch in the library's static per-device array: allocates
    nothing (not even a temporary workspace)."""
    _check(load_library().hstu_attn_fwd_noalloc(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(u),
        float(ln_eps), _ptr(out), _stream(stream)))


def hstu_attn_bwd(plan: Plan, args: HstuAttnArgs, q, k, v, dout, dq, dk, dv, drab_pos=None,
                  drab_ts=None, ws=None, stream=None) -> None:
    ws, nbytes = _workspace(plan, OP_BWD, 0, ws, q.device, stream)
    _check(load_library().hstu_attn_bwd(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drab_pos), _ptr(drab_ts), _ptr(ws), nbytes,
        _stream(stream)))


def hstu_attn_bwd_dkdv(plan: Plan, args: HstuAttnArgs, q, k, v, dout, dk, dv, ws=None,
                       stream=None) -> None:
    """dK, dV; with ws (hstu_workspace_bytes(plan, OP_BWD) bytes) also stores dS and the
    bias-table gradients there for hstu_attn_bwd_dq."""
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load_library().hstu_attn_bwd_dkdv(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
        _ptr(dk), _ptr(dv), _ptr(ws), nbytes, _stream(stream)))


def hstu_attn_bwd_dq(plan: Plan, args: HstuAttnArgs, q, k, v, dout, dq, drab_pos=None,
                     drab_ts=None, ws=None, stream=None) -> None:
    """dQ and the bias-table gradients; with ws, reads the dS and copies out the gradients that
    hstu_attn_bwd_dkdv left in the same ws, else recomputes S and dP and sums the gradients."""
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load_library().hstu_attn_bwd_dq(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
        _ptr(dq), _ptr(drab_pos), _ptr(drab_ts), _ptr(ws), nbytes, _stream(stream)))


def hstu_layer_fwd(plan: Plan, args: HstuAttnArgs, d_model: int, x, w1, w2, y,
                   ln_eps: float = 1e-5, ws=None, stream=None) -> None:
    ws, nbytes = _workspace(plan, OP_LAYER, d_model, ws, x.device, stream)
    _check(load_library().hstu_layer_fwd(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), int(d_model), _ptr(x), _ptr(w1),
        _ptr(w2), float(ln_eps), _ptr(y), _ptr(ws), nbytes, _stream(stream)))


def hstu_layer_bwd(plan: Plan, args: HstuAttnArgs, d_model: int, x, w1, w2, dy, dx, dw1, dw2,
                   drab_pos=None, drab_ts=None, ln_eps: float = 1e-5, ws=None,
                   stream=None) -> None:
    ws, nbytes = _workspace(plan, OP_LAYER_BWD, d_model, ws, x.device, stream)
    _check(load_library().hstu_layer_bwd(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), int(d_model), _ptr(x), _ptr(w1),
        _ptr(w2), _ptr(dy), float(ln_eps), _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(drab_pos),
        _ptr(drab_ts), _ptr(ws), nbytes, _stream(stream)))


def hstu_attn_fwd_cached(plan: Plan, args: HstuAttnArgs, q, k, v, k_cache, v_cache,
                         cache_timestamps, out, ws=None, stream=None) -> None:
    ws, nbytes = _workspace(plan, OP_CACHED, 0, ws, q.device, stream)
    _check(load_library().hstu_attn_fwd_cached(
        ctypes.c_void_p(plan.handle), ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v),
        _ptr(k_cache), _ptr(v_cache), _ptr(cache_timestamps), _ptr(out), _ptr(ws), nbytes,
        _stream(stream)))


def hstu_jagged_select(src_offsets, dst_offsets, src, dst, keep_start=None, stream=None) -> None:
    """Stochastic Length compaction: device int64 offsets (B + 1), contiguous src / dst tensors
    whose first dimension is the token; keep_start (device int64 [B]) or None for the last
    rows of each sequence."""
    B = int(src_offsets.numel()) - 1
    row_bytes = int(src[0].numel() * src.element_size()) if src.shape[0] else \
        int(np.prod(src.shape[1:], dtype=np.int64)) * src.element_size()
    _check(load_library().hstu_jagged_select(
        B, _ptr(src_offsets), int(src.shape[0]), _ptr(dst_offsets), int(dst.shape[0]),
        _ptr(keep_start), row_bytes, _ptr(src), _ptr(dst), _stream(stream)))
