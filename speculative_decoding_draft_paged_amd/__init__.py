"""Python binding of the blockattn C ABI (``include/blockattn.h``).

Argument marshalling only: every step of the attention runs in the gfx950
kernels of ``libblockattn.so``. PyTorch supplies device memory and streams.
There is no fallback: if the library is not built, importing the entry points
raises.

The functions carry the C names. Tensors are passed by pointer after a check
that their dtype, device, contiguity and element count match the plan's
shapes, so a mismatched buffer is refused on the host instead of reaching a
kernel.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libblockattn.so")

BLOCKATTN_OK = 0
BLOCKATTN_ERR_INVALID_ARGUMENT = 1
BLOCKATTN_ERR_UNSUPPORTED = 2
BLOCKATTN_ERR_WORKSPACE_TOO_SMALL = 3
BLOCKATTN_ERR_PLAN_MISMATCH = 4
BLOCKATTN_ERR_HIP = 5
BLOCKATTN_KV_BF16 = 0
BLOCKATTN_KV_FP8_E4M3 = 1
BLOCKATTN_COMBINE_AUTO = 0
BLOCKATTN_COMBINE_KERNEL = 1
BLOCKATTN_COMBINE_LAST_ARRIVER = 2
COMBINE_MODES = {"auto": 0, "kernel": 1, "last_arriver": 2}
BLOCKATTN_SCRATCH_BYTES = 32 << 20
BLOCKATTN_INPUT_BAD_LENGTH = 1
BLOCKATTN_INPUT_BAD_PAGE = 2

EXPORTED = (
    "blockattn_workspace_size",
    "blockattn_plan",
    "blockattn_forward",
    "blockattn_windowed_forward",
    "blockattn_forward_block",
    "blockattn_forward_scratch",
    "blockattn_merge",
    "blockattn_plan_info",
    "blockattn_plan_set_profile_events",
    "blockattn_plan_set_phase_trace",
    "blockattn_input_errors",
    "blockattn_stream_read",
    "blockattn_plan_destroy",
    "blockattn_last_error",
)


class blockattn_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("page_table_stride", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("splits_override", ctypes.c_int32),
        ("waves_override", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("combine_mode", ctypes.c_int32),
    ]


class blockattn_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("units", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("merge_active", ctypes.c_int32),
        ("waves_per_unit", ctypes.c_int32),
        ("token_groups", ctypes.c_int32),
        ("row_waves", ctypes.c_int32),
        ("uploaded", ctypes.c_int32),
        ("combine_launch", ctypes.c_int32),
        ("shared_tiles", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("fused_combine", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class BlockAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"blockattn status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library():
    """Load libblockattn.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback path)")
    # Load torch's HIP runtime first so the library binds to the same runtime instance
    # (same soname): streams, events and device pointers are then shared.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    pp = ctypes.POINTER(blockattn_params)
    lib.blockattn_workspace_size.argtypes = [pp, i32p, ctypes.POINTER(ctypes.c_size_t)]
    lib.blockattn_plan.argtypes = [pp, i32p, vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
    fwd = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.blockattn_forward.argtypes = fwd
    lib.blockattn_windowed_forward.argtypes = fwd
    lib.blockattn_forward_block.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
    lib.blockattn_forward_scratch.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.blockattn_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp, vp]
    lib.blockattn_plan_info.argtypes = [vp, ctypes.POINTER(blockattn_plan_info_t)]
    lib.blockattn_plan_set_profile_events.argtypes = [vp, vp, vp]
    lib.blockattn_input_errors.argtypes = [vp, vp, vp, i32p]
    lib.blockattn_plan_set_phase_trace.argtypes = [vp, vp, ctypes.c_size_t]
    lib.blockattn_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int32, vp]
    lib.blockattn_plan_destroy.argtypes = [vp]
    lib.blockattn_plan_destroy.restype = None
    lib.blockattn_last_error.restype = ctypes.c_char_p
    for name in ("blockattn_workspace_size", "blockattn_plan", "blockattn_forward", "blockattn_windowed_forward",
                 "blockattn_forward_block", "blockattn_forward_scratch", "blockattn_merge", "blockattn_plan_info",
                 "blockattn_plan_set_profile_events", "blockattn_plan_set_phase_trace", "blockattn_input_errors",
                 "blockattn_stream_read"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def blockattn_last_error() -> str:
    return load_library().blockattn_last_error().decode()


def _check(status: int):
    if status != BLOCKATTN_OK:
        raise BlockAttnError(status, blockattn_last_error())


KV_DTYPES = {"bf16": BLOCKATTN_KV_BF16, "fp8_e4m3": BLOCKATTN_KV_FP8_E4M3}


def make_params(*, batch, block_size, num_q_heads, num_kv_heads, head_dim, page_size, page_table_stride, num_pages,
                sm_scale, window_left=-1, window_right=-1, splits_override=0, waves_override=0, kv_dtype="bf16",
                k_scale=1.0, v_scale=1.0, combine="auto") -> blockattn_params:
    code = KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    mode = COMBINE_MODES[combine] if isinstance(combine, str) else int(combine)
    return blockattn_params(batch, block_size, num_q_heads, num_kv_heads, head_dim, page_size, page_table_stride,
                            num_pages, window_left, window_right, float(sm_scale), splits_override, waves_override,
                            code, float(k_scale), float(v_scale), mode)


def _host_lens(seq_lens_host):
    if hasattr(seq_lens_host, "detach"):
        seq_lens_host = seq_lens_host.detach().cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def blockattn_workspace_size(params: blockattn_params, seq_lens_host) -> int:
    lib = load_library()
    arr, p = _host_lens(seq_lens_host)
    if arr.shape[0] < params.batch:
        raise ValueError("seq_lens_host has fewer than batch entries")
    out = ctypes.c_size_t(0)
    _check(lib.blockattn_workspace_size(ctypes.byref(params), p, ctypes.byref(out)))
    return int(out.value)


class Plan:
    """Owns a blockattn plan handle; remembers its params for the host-side buffer checks."""

    def __init__(self, handle, params: blockattn_params, workspace):
        self.handle = handle
        self.params = params
        self.workspace = workspace

    def info(self) -> dict:
        return blockattn_plan_info(self)

    def destroy(self):
        if self.handle:
            blockattn_plan_destroy(self)

    def __del__(self):
        try:
            self.destroy()
        except Exception:  # interpreter shutdown
            pass


def blockattn_plan(params: blockattn_params, seq_lens_host, workspace=None, workspace_bytes=None,
                   stream=None) -> Plan:
    """Validate and plan; with a workspace tensor, enqueue the work-list upload on the stream."""
    lib = load_library()
    arr, p = _host_lens(seq_lens_host)
    if arr.shape[0] < params.batch:
        raise ValueError("seq_lens_host has fewer than batch entries")
    handle = ctypes.c_void_p(0)
    if workspace is None:
        _check(lib.blockattn_plan(ctypes.byref(params), p, None, 0, None, ctypes.byref(handle)))
    else:
        nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        _check(lib.blockattn_plan(ctypes.byref(params), p, ctypes.c_void_p(_ptr(workspace)), nbytes,
                                  ctypes.c_void_p(_stream(stream)), ctypes.byref(handle)))
    return Plan(handle.value, params, workspace)


def blockattn_plan_info(plan: Plan) -> dict:
    info = blockattn_plan_info_t()
    _check(load_library().blockattn_plan_info(ctypes.c_void_p(plan.handle), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in blockattn_plan_info_t._fields_}


def blockattn_plan_set_profile_events(plan: Plan, before, after):
    """Record raw hipEvent_t handles (ints) around the partial kernel of later forwards; None stops."""
    _check(load_library().blockattn_plan_set_profile_events(ctypes.c_void_p(plan.handle), ctypes.c_void_p(before),
                                                            ctypes.c_void_p(after)))


def blockattn_plan_set_phase_trace(plan: Plan, trace):
    """Per-unit phase timestamps of later forwards into `trace` (int64 device tensor of units * 8); None stops."""
    if trace is None:
        _check(load_library().blockattn_plan_set_phase_trace(ctypes.c_void_p(plan.handle), None, 0))
        return
    if not trace.is_cuda or not trace.is_contiguous():
        raise ValueError("trace must be a contiguous device tensor")
    _check(load_library().blockattn_plan_set_phase_trace(ctypes.c_void_p(plan.handle), ctypes.c_void_p(_ptr(trace)),
                                                         trace.numel() * trace.element_size()))


def blockattn_input_errors(plan: Plan, workspace, stream=None) -> int:
    """Out-of-range device inputs met since the last call (BLOCKATTN_INPUT_* bits); clears the record."""
    flags = ctypes.c_int32(0)
    _check(load_library().blockattn_input_errors(ctypes.c_void_p(plan.handle), ctypes.c_void_p(_ptr(workspace)),
                                                 ctypes.c_void_p(_stream(stream)), ctypes.byref(flags)))
    return int(flags.value)


def blockattn_stream_read(src, result, workgroups=0, stream=None):
    """Read-only streaming reference over the bytes of `src` (a device tensor); XOR fold into `result`."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _expect("result", result, 1, ("int32", "uint32"))
    vp = ctypes.c_void_p
    _check(load_library().blockattn_stream_read(vp(_ptr(src)), src.numel() * src.element_size(), vp(_ptr(result)),
                                                ctypes.c_int32(workgroups), vp(_stream(stream))))


def blockattn_plan_destroy(plan: Plan):
    if plan.handle:
        load_library().blockattn_plan_destroy(ctypes.c_void_p(plan.handle))
        plan.handle = None


def _expect(name, t, numel, dtypes):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements; expected {numel}")


def _check_buffers(plan: Plan, q, k_cache, v_cache, page_table, seq_lens, out, lse):
    p = plan.params
    rows = p.batch * p.block_size * p.num_q_heads
    _expect("q", q, rows * p.head_dim, ("bfloat16", "int16", "uint16"))
    _expect("out", out, rows * p.head_dim, ("bfloat16", "int16", "uint16"))
    pool = p.num_pages * p.num_kv_heads * p.page_size * p.head_dim
    kv = ("uint8", "int8", "float8_e4m3fn") if p.kv_dtype == BLOCKATTN_KV_FP8_E4M3 else ("bfloat16", "int16", "uint16")
    _expect("k_cache", k_cache, pool, kv)
    _expect("v_cache", v_cache, pool, kv)
    _expect("page_table", page_table, p.batch * p.page_table_stride, ("int32",))
    _expect("seq_lens", seq_lens, p.batch, ("int32",))
    if lse is not None:
        _expect("lse", lse, rows, ("float32",))


def _forward(fn_name, plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse, stream):
    _check_buffers(plan, q, k_cache, v_cache, page_table, seq_lens, out, lse)
    fn = getattr(load_library(), fn_name)
    vp = ctypes.c_void_p
    _check(fn(vp(plan.handle), vp(_ptr(q)), vp(_ptr(k_cache)), vp(_ptr(v_cache)), vp(_ptr(page_table)),
              vp(_ptr(seq_lens)), vp(_ptr(workspace)), vp(_ptr(out)), vp(_ptr(lse)), vp(_stream(stream))))


def blockattn_forward(plan: Plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse=None, stream=None):
    """Non-causal unwindowed block attention (launch only)."""
    _forward("blockattn_forward", plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse, stream)


def blockattn_windowed_forward(plan: Plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse,
                               stream=None):
    """Non-causal windowed block attention: causal windowed decode + future-key merge (launch only)."""
    _forward("blockattn_windowed_forward", plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse,
             stream)


def blockattn_forward_scratch(plan: Plan, q, k_cache, v_cache, page_table, seq_lens, out, lse=None, stream=None):
    """Either form (the plan's kind) with no workspace: the library's per-GPU scratch array holds the
    work list and partials (for callers that cannot allocate; overlapping calls on one GPU race)."""
    _check_buffers(plan, q, k_cache, v_cache, page_table, seq_lens, out, lse)
    vp = ctypes.c_void_p
    _check(load_library().blockattn_forward_scratch(
        vp(plan.handle), vp(_ptr(q)), vp(_ptr(k_cache)), vp(_ptr(v_cache)), vp(_ptr(page_table)), vp(_ptr(seq_lens)),
        vp(_ptr(out)), vp(_ptr(lse)), vp(_stream(stream))))


def blockattn_forward_block(plan: Plan, q, k_block, v_block, k_cache, v_cache, page_table, seq_lens, workspace, out,
                            lse=None, append=False, stream=None):
    """Block attention with the block's K/V from dense bf16 [B, K, Hkv, D] arrays; optionally append them."""
    _check_buffers(plan, q, k_cache, v_cache, page_table, seq_lens, out, lse)
    p = plan.params
    blk = p.batch * p.block_size * p.num_kv_heads * p.head_dim
    _expect("k_block", k_block, blk, ("bfloat16", "int16", "uint16"))
    _expect("v_block", v_block, blk, ("bfloat16", "int16", "uint16"))
    vp = ctypes.c_void_p
    _check(load_library().blockattn_forward_block(
        vp(plan.handle), vp(_ptr(q)), vp(_ptr(k_block)), vp(_ptr(v_block)), vp(_ptr(k_cache)), vp(_ptr(v_cache)),
        vp(_ptr(page_table)), vp(_ptr(seq_lens)), vp(_ptr(workspace)), vp(_ptr(out)), vp(_ptr(lse)),
        ctypes.c_int32(1 if append else 0), vp(_stream(stream))))


def blockattn_merge(part_out, part_lse, out, lse=None, stream=None):
    """G-way LSE merge: part_out bf16 [G, ..., D] and part_lse fp32 [G, ...] (base 2) into out [..., D] and lse."""
    if part_out is None or part_lse is None:
        raise ValueError("part_out and part_lse are required")
    G = int(part_lse.shape[0])
    rows = int(part_lse[0].numel()) if G > 0 else 0
    D = int(part_out.shape[-1])
    _expect("part_out", part_out, G * rows * D, ("bfloat16", "int16", "uint16"))
    _expect("part_lse", part_lse, G * rows, ("float32",))
    _expect("out", out, rows * D, ("bfloat16", "int16", "uint16"))
    if lse is not None:
        _expect("lse", lse, rows, ("float32",))
    vp = ctypes.c_void_p
    _check(load_library().blockattn_merge(ctypes.c_int32(G), ctypes.c_int64(rows), ctypes.c_int32(D),
                                          vp(_ptr(part_out)), vp(_ptr(part_lse)), vp(_ptr(out)), vp(_ptr(lse)),
                                          vp(_stream(stream))))
