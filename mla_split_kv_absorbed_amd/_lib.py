"""Thin ctypes binding of libmla_decode.so (the C ABI in include/mla_decode.h).

Argument marshalling only: every step of the decode path runs in the
library's HIP kernels. PyTorch supplies device memory (data_ptr) and the
stream handle. If the library is missing, every call raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime the library then shares)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")

MLA_F32, MLA_BF16, MLA_F16 = 0, 1, 2
MLA_MASK_NONE, MLA_MASK_CAUSAL_WINDOW = 0, 1
MLA_FLAG_FORCE_SIMPLE = 1
MLA_OK = 0
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_RANGE", -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_UNSUPPORTED",
          -7: "MLA_ERR_HIP", -8: "MLA_ERR_ALIAS"}

DT_CODE = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16, torch.float16: MLA_F16}
NAME_CODE = {"f32": MLA_F32, "bf16": MLA_BF16, "f16": MLA_F16}
CODE_TORCH = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16, MLA_F16: torch.float16}

D_C, D_R, D_ROW, D_NOPE, D_V = 512, 64, 576, 128, 128


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class PartialArgs(ctypes.Structure):
    _fields_ = [
        ("q_lat", ctypes.c_void_p), ("q_rope", ctypes.c_void_p), ("q_dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("S", ctypes.c_int), ("H", ctypes.c_int),
        ("kv", ctypes.c_void_p), ("kv_dtype", ctypes.c_int),
        ("block_size", ctypes.c_int), ("block_table", ctypes.c_void_p),
        ("max_blocks", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("kv_seq_stride", ctypes.c_int),
        ("P", ctypes.c_int), ("range_start", ctypes.c_void_p), ("range_end", ctypes.c_void_p),
        ("mask", ctypes.c_int), ("scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
        ("lse", ctypes.c_void_p), ("lse_dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_splits", ctypes.c_int), ("flags", ctypes.c_uint),
        ("plan", ctypes.c_void_p), ("plan_chunks", ctypes.c_int),
        ("plan_split_units", ctypes.c_int),
    ]


class SplitInfo(ctypes.Structure):
    _fields_ = [
        ("matrix_path", ctypes.c_int), ("chunk_tiles", ctypes.c_int), ("chunks", ctypes.c_int),
        ("split_ranges", ctypes.c_int), ("split_chunks", ctypes.c_int),
        ("equal_splits", ctypes.c_int), ("max_chunks", ctypes.c_int),
        ("max_split_slots", ctypes.c_int),
    ]


class PrologueArgs(ctypes.Structure):
    _fields_ = [
        ("q_nope", ctypes.c_void_p), ("q_pe", ctypes.c_void_p), ("w_uk", ctypes.c_void_p),
        ("kv_new", ctypes.c_void_p), ("positions", ctypes.c_void_p), ("dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("S", ctypes.c_int), ("H", ctypes.c_int),
        ("rope_theta", ctypes.c_float),
        ("kv", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("block_size", ctypes.c_int), ("max_blocks", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("kv_seq_stride", ctypes.c_int),
        ("q_lat", ctypes.c_void_p), ("q_rope", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m mla_split_kv_absorbed_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.mla_abi_version.restype = ci
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_status_string.argtypes = [ci]
        L.mla_decode_partial_workspace_size.restype = ctypes.c_size_t
        L.mla_decode_partial_workspace_size.argtypes = [ctypes.POINTER(PartialArgs)]
        L.mla_decode_partial.restype = ci
        L.mla_decode_partial.argtypes = [ctypes.POINTER(PartialArgs), vp]
        L.mla_decode_partial_pair.restype = ci
        L.mla_decode_partial_pair.argtypes = [ctypes.POINTER(PartialArgs),
                                              ctypes.POINTER(PartialArgs), vp]
        L.mla_q_absorb.restype = ci
        L.mla_q_absorb.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        L.mla_vup.restype = ci
        L.mla_vup.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        L.mla_lse_combine.restype = ci
        L.mla_lse_combine.argtypes = [vp, vp, ci, ci, ci, vp, vp, ci, ci, vp, ci, vp, vp]
        L.mla_combine_vup.restype = ci
        L.mla_combine_vup.argtypes = [vp, vp, ci, ci, ci, vp, vp, ci, ci, vp, ci, vp, vp, vp,
                                      vp]
        L.mla_decode_prologue.restype = ci
        L.mla_decode_prologue.argtypes = [ctypes.POINTER(PrologueArgs), vp]
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.mla_decode_partial_plan.restype = ci
        L.mla_decode_partial_plan.argtypes = [ctypes.POINTER(PartialArgs), i32p, i32p,
                                              ctypes.POINTER(SplitInfo)]
        L.mla_decode_partial_noalloc.restype = ci
        L.mla_decode_partial_noalloc.argtypes = [ctypes.POINTER(PartialArgs), vp]
        L.mla_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.mla_noalloc_scratch_bytes.argtypes = []
        L.mla_cut_ranges.restype = ci
        L.mla_cut_ranges.argtypes = [i32p, i32p, ci, ci, i32p, i32p]
        L.mla_decode_partial_plan_words.restype = ctypes.c_size_t
        L.mla_decode_partial_plan_words.argtypes = [ctypes.POINTER(PartialArgs)]
        L.mla_decode_partial_make_plan.restype = ci
        L.mla_decode_partial_make_plan.argtypes = [ctypes.POINTER(PartialArgs), i32p, i32p, i32p,
                                                   ctypes.c_size_t, ctypes.POINTER(SplitInfo)]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MLAError(status, what)


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def mla_abi_version() -> int:
    return lib().mla_abi_version()


def partial_args(q_lat, q_rope, kv, range_start, range_end, out, lse, *, B, S, H,
                 block_table=None, block_size=0, num_blocks=0, kv_seq_stride=0,
                 mask=MLA_MASK_NONE, scale, workspace=None, num_splits=0, flags=0) -> PartialArgs:
    a = PartialArgs()
    a.q_lat, a.q_rope = _ptr(q_lat), _ptr(q_rope)
    a.q_dtype = DT_CODE[q_lat.dtype]
    a.B, a.S, a.H = B, S, H
    a.kv, a.kv_dtype = _ptr(kv), DT_CODE[kv.dtype]
    a.block_size = block_size
    a.block_table = _ptr(block_table)
    a.max_blocks = block_table.shape[1] if block_table is not None else 0
    a.num_blocks = num_blocks
    a.kv_seq_stride = kv_seq_stride
    a.P = range_start.shape[0]
    a.range_start, a.range_end = _ptr(range_start), _ptr(range_end)
    a.mask, a.scale = mask, scale
    a.out, a.out_dtype = _ptr(out), DT_CODE[out.dtype]
    a.lse, a.lse_dtype = _ptr(lse), DT_CODE[lse.dtype]
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.num_splits, a.flags = num_splits, flags
    return a


def mla_decode_partial_workspace_size(a: PartialArgs) -> int:
    n = lib().mla_decode_partial_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise MLAError(-2, "mla_decode_partial_workspace_size")
    return n


def mla_decode_partial(a: PartialArgs, stream=None):
    _check(lib().mla_decode_partial(ctypes.byref(a), _stream(stream)), "mla_decode_partial")


def mla_decode_partial_pair(hist: PartialArgs, cur: PartialArgs, stream=None):
    _check(lib().mla_decode_partial_pair(ctypes.byref(hist), ctypes.byref(cur), _stream(stream)),
           "mla_decode_partial_pair")


def _host_i32(a):
    import numpy as np
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def mla_decode_partial_plan(a: PartialArgs, range_start, range_end) -> SplitInfo:
    """The split plan mla_decode_partial evaluates for `a`, from host copies
    of its [P][B] ranges (numpy or CPU arrays)."""
    rs, re_ = _host_i32(range_start), _host_i32(range_end)
    if rs.size != a.P * a.B or re_.size != a.P * a.B:
        raise ValueError("ranges must hold P x B entries")
    info = SplitInfo()
    _check(lib().mla_decode_partial_plan(ctypes.byref(a), _i32p(rs), _i32p(re_),
                                         ctypes.byref(info)), "mla_decode_partial_plan")
    return info


def mla_decode_partial_plan_words(a: PartialArgs) -> int:
    return lib().mla_decode_partial_plan_words(ctypes.byref(a))


def mla_decode_partial_make_plan(a: PartialArgs, range_start, range_end):
    """The plan mla_decode_partial evaluates on the device, built on the host
    from host copies of the [P][B] ranges: (int32 numpy table, SplitInfo).
    The caller copies the table to device memory and sets a.plan,
    a.plan_chunks = info.chunks, a.plan_split_units = info.split_ranges."""
    import numpy as np
    rs, re_ = _host_i32(range_start), _host_i32(range_end)
    if rs.size != a.P * a.B or re_.size != a.P * a.B:
        raise ValueError("ranges must hold P x B entries")
    words = mla_decode_partial_plan_words(a)  # 0: invalid arguments or the plain kernel
    table = np.zeros(max(words, 1), np.int32)
    info = SplitInfo()
    _check(lib().mla_decode_partial_make_plan(ctypes.byref(a), _i32p(rs), _i32p(re_),
                                              _i32p(table), words, ctypes.byref(info)),
           "mla_decode_partial_make_plan")
    return table, info


def mla_cut_ranges(range_start, range_end, k: int):
    """Pieces [k][n] of the n ranges that num_splits = k cuts (host arrays)."""
    import numpy as np
    rs, re_ = _host_i32(range_start).ravel(), _host_i32(range_end).ravel()
    n = rs.size
    ps = np.empty((k, n), np.int32)
    pe = np.empty((k, n), np.int32)
    _check(lib().mla_cut_ranges(_i32p(rs), _i32p(re_), n, k, _i32p(ps), _i32p(pe)),
           "mla_cut_ranges")
    return ps, pe


def mla_decode_partial_noalloc(a: PartialArgs, stream=None):
    """mla_decode_partial with the library's device scratch as workspace
    (a.workspace is ignored)."""
    _check(lib().mla_decode_partial_noalloc(ctypes.byref(a), _stream(stream)),
           "mla_decode_partial_noalloc")


def mla_noalloc_scratch_bytes() -> int:
    return lib().mla_noalloc_scratch_bytes()


def mla_q_absorb(q_nope, w_uk, q_lat, stream=None):
    T, H = q_nope.shape[0], q_nope.shape[1]
    _check(lib().mla_q_absorb(_ptr(q_nope), _ptr(w_uk), _ptr(q_lat), T, H, DT_CODE[q_nope.dtype],
                              _stream(stream)), "mla_q_absorb")


def mla_vup(x, w_uv, out, stream=None):
    T, H = x.shape[0], x.shape[1]
    _check(lib().mla_vup(_ptr(x), _ptr(w_uv), _ptr(out), T, H, DT_CODE[x.dtype],
                         _stream(stream)), "mla_vup")


def mla_lse_combine(parts_out, parts_lse, out, lse_out=None, local_out=None, local_lse=None,
                    stream=None):
    """parts_out [P][T][H][512] (P may be 0 / None with a local part)."""
    ref = parts_out if parts_out is not None else local_out
    refl = parts_lse if parts_lse is not None else local_lse
    P = parts_out.shape[0] if parts_out is not None else 0
    T, H = out.shape[0], out.shape[1]
    _check(lib().mla_lse_combine(_ptr(parts_out), _ptr(parts_lse), P, DT_CODE[ref.dtype],
                                 DT_CODE[refl.dtype], _ptr(local_out), _ptr(local_lse), T, H,
                                 _ptr(out), DT_CODE[out.dtype], _ptr(lse_out), _stream(stream)),
           "mla_lse_combine")


def mla_combine_vup(parts_out, parts_lse, w_uv, out, lse_out=None, lat_out=None,
                    local_out=None, local_lse=None, stream=None):
    """parts_out [P][T][H][512] (P may be 0 / None with a local part),
    w_uv [H][512][128], out [T][H][128] in the compute dtype."""
    ref = parts_out if parts_out is not None else local_out
    refl = parts_lse if parts_lse is not None else local_lse
    P = parts_out.shape[0] if parts_out is not None else 0
    T, H = out.shape[0], out.shape[1]
    _check(lib().mla_combine_vup(_ptr(parts_out), _ptr(parts_lse), P, DT_CODE[ref.dtype],
                                 DT_CODE[refl.dtype], _ptr(local_out), _ptr(local_lse), T, H,
                                 _ptr(w_uv), DT_CODE[out.dtype], _ptr(out), _ptr(lse_out),
                                 _ptr(lat_out), _stream(stream)),
           "mla_combine_vup")


def prologue_args(q_nope, q_pe, w_uk, kv_new, positions, kv, q_lat, q_rope, *, B, S,
                  rope_theta=10000.0, block_table=None, block_size=0, num_blocks=0,
                  kv_seq_stride=0) -> PrologueArgs:
    a = PrologueArgs()
    a.q_nope, a.q_pe, a.w_uk = _ptr(q_nope), _ptr(q_pe), _ptr(w_uk)
    a.kv_new, a.positions = _ptr(kv_new), _ptr(positions)
    a.dtype = DT_CODE[q_nope.dtype]
    a.B, a.S, a.H = B, S, q_nope.shape[1]
    a.rope_theta = rope_theta
    a.kv, a.block_table = _ptr(kv), _ptr(block_table)
    a.block_size = block_size
    a.max_blocks = block_table.shape[1] if block_table is not None else 0
    a.num_blocks = num_blocks
    a.kv_seq_stride = kv_seq_stride
    a.q_lat, a.q_rope = _ptr(q_lat), _ptr(q_rope)
    return a


def mla_decode_prologue(a: PrologueArgs, stream=None):
    _check(lib().mla_decode_prologue(ctypes.byref(a), _stream(stream)), "mla_decode_prologue")
