"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import math
import os
import re
import subprocess
import sys

import pytest

from mla_split_kv_absorbed_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libmla_decode.so not built")

FAKE = 0x10000  # non-NULL, never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"mla_decode_partial", "mla_lse_combine", "mla_vup", "mla_q_absorb",
            "mla_decode_partial_workspace_size", "mla_status_string",
            "mla_abi_version"} <= set(names)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings():
    assert L.mla_abi_version() == 2
    for code, name in L.STATUS.items():
        assert L.mla_status_string(code).startswith(name)
    assert L.mla_status_string(12345) == "unknown status"


def base_args(**over):
    a = L.PartialArgs()
    a.q_lat, a.q_rope, a.kv = FAKE, FAKE + 0x10000000, FAKE + 0x20000000
    a.q_dtype = a.kv_dtype = L.MLA_BF16
    a.B, a.S, a.H = 2, 1, 128
    a.block_size, a.block_table = 32, FAKE + 0x30000000
    a.max_blocks, a.num_blocks = 4, 8
    a.P = 2
    a.range_start, a.range_end = FAKE + 0x40000000, FAKE + 0x40001000
    a.mask, a.scale = L.MLA_MASK_NONE, 1.0 / math.sqrt(192)
    a.out, a.out_dtype = FAKE + 0x50000000, L.MLA_BF16
    a.lse, a.lse_dtype = FAKE + 0x60000000, L.MLA_F32
    a.workspace, a.workspace_bytes = FAKE + 0x70000000, 1 << 40
    for k, v in over.items():
        setattr(a, k, v)
    return a


def call(a):
    return L.lib().mla_decode_partial(ctypes.byref(a), None)


@pytest.mark.parametrize("over,code", [
    (dict(q_lat=None), -1), (dict(kv=None), -1), (dict(out=None), -1),
    (dict(range_end=None), -1), (dict(block_table=None), -1),
    (dict(q_dtype=7), -3), (dict(out_dtype=-1), -3), (dict(kv_dtype=L.MLA_F16), -3),
    (dict(P=0), -2), (dict(B=0), -2), (dict(H=0), -2), (dict(S=0), -2),
    (dict(S=65), -6), (dict(block_size=-1), -2), (dict(max_blocks=0), -2),
    (dict(num_blocks=0), -2), (dict(block_size=0), -2),
    (dict(block_size=0, block_table=None, kv_seq_stride=0), -2),
    (dict(mask=5), -4), (dict(scale=float("nan")), -4), (dict(num_splits=-1), -4),
    (dict(flags=0x80), -4),
    (dict(out=FAKE), -8), (dict(lse=FAKE + 0x20000000 + 64), -8),
    (dict(workspace=FAKE + 0x50000000), -8),
    # row tensors must be 16-byte aligned (LSE / int32 arrays need not be)
    (dict(q_lat=FAKE + 8), -4), (dict(kv=FAKE + 0x20000000 + 4), -4),
    (dict(out=FAKE + 0x50000000 + 2), -4), (dict(workspace=FAKE + 0x70000000 + 8), -4),
])
def test_partial_validation(over, code):
    assert call(base_args(**over)) == code


def test_workspace_checks():
    a = base_args()
    need = L.lib().mla_decode_partial_workspace_size(ctypes.byref(a))
    assert 0 < need < (1 << 40)
    assert call(base_args(workspace_bytes=need - 1)) == -5
    assert call(base_args(workspace=None)) == -5
    # the plain kernel needs no workspace; invalid arguments have no size
    assert L.lib().mla_decode_partial_workspace_size(
        ctypes.byref(base_args(flags=L.MLA_FLAG_FORCE_SIMPLE))) == 0
    assert L.lib().mla_decode_partial_workspace_size(ctypes.byref(base_args(P=0))) == \
        ctypes.c_size_t(-1).value
    # a pure function of the sizes: more splits never need less
    s1 = L.lib().mla_decode_partial_workspace_size(ctypes.byref(base_args(num_splits=1)))
    s8 = L.lib().mla_decode_partial_workspace_size(ctypes.byref(base_args(num_splits=8)))
    assert s8 >= s1


def test_combine_vup_absorb_validation():
    lib = L.lib()
    c = lib.mla_lse_combine
    # both local pointers or none
    assert c(FAKE, FAKE + 4096, 2, 1, 0, FAKE * 8, None, 4, 8, FAKE * 16, 1, None, None) == -1
    assert c(None, None, 0, 1, 0, None, None, 4, 8, FAKE * 16, 1, None, None) == -2
    assert c(FAKE, FAKE * 4, 2, 9, 0, None, None, 4, 8, FAKE * 16, 1, None, None) == -3
    assert c(FAKE, FAKE * 4, 2, 1, 0, None, None, 0, 8, FAKE * 16, 1, None, None) == -2
    assert c(FAKE, FAKE * 4, 2, 1, 0, None, None, 4, 8, FAKE, 1, None, None) == -8
    assert c(FAKE, FAKE * 4, 2, 1, 0, None, None, 4, 8, None, 1, None, None) == -1
    assert lib.mla_vup(None, FAKE, FAKE * 2, 4, 8, 1, None) == -1
    assert lib.mla_vup(FAKE, FAKE * 64, FAKE * 128, 0, 8, 1, None) == -2
    assert lib.mla_vup(FAKE, FAKE * 64, FAKE * 128, 4, 8, 3, None) == -3
    assert lib.mla_vup(FAKE, FAKE * 64, FAKE, 4, 8, 1, None) == -8
    assert lib.mla_q_absorb(FAKE, None, FAKE * 2, 4, 8, 1, None) == -1
    assert lib.mla_q_absorb(FAKE, FAKE * 64, FAKE * 128, 4, 0, 1, None) == -2
    assert lib.mla_q_absorb(FAKE, FAKE * 64, FAKE + 100, 4, 8, 1, None) == -8
    assert lib.mla_q_absorb(FAKE, FAKE * 64 + 8, FAKE * 128, 4, 8, 1, None) == -4
    assert lib.mla_vup(FAKE + 4, FAKE * 64, FAKE * 128, 4, 8, 1, None) == -4
    assert c(FAKE, FAKE * 4, 2, 1, 0, None, None, 4, 8, FAKE * 16 + 8, 1, None, None) == -4


def test_fused_combine_vup_validation():
    cv = L.lib().mla_combine_vup
    # parts [2][4][8][512] bf16 at FAKE, LSEs at 4 FAKE, W_UV [8][512][128] at
    # 64 FAKE, out [4][8][128] at 128 FAKE, lat_out at 256 FAKE, lse_out at 512 FAKE
    P, W, O, X, LS = FAKE * 4, FAKE * 64, FAKE * 128, FAKE * 256, FAKE * 512

    def call(**over):
        a = dict(parts=FAKE, lse=P, n=2, pdt=1, ldt=0, lo=None, ll=None, T=4, H=8, w=W, dt=1,
                 out=O, lse_out=LS, lat=X)
        a.update(over)
        return cv(a["parts"], a["lse"], a["n"], a["pdt"], a["ldt"], a["lo"], a["ll"], a["T"],
                  a["H"], a["w"], a["dt"], a["out"], a["lse_out"], a["lat"], None)
    assert call(out=None) == -1
    assert call(w=None) == -1
    assert call(lo=FAKE * 1024) == -1          # local part without its LSE
    assert call(parts=None) == -1
    assert call(pdt=9) == -3
    assert call(dt=7) == -3
    assert call(T=0) == -2
    assert call(H=0) == -2
    assert call(n=0) == -2                     # no part at all
    assert call(n=-1) == -2
    assert call(dt=0) == -6                    # fp32: the two separate calls
    assert call(out=FAKE + 64) == -8           # out overlaps the parts
    assert call(lat=W + 4096) == -8            # merged latent overlaps W_UV
    assert call(lse_out=O + 64) == -8          # the two outputs overlap
    assert call(w=W + 8) == -4                 # W_UV not 16-byte aligned
    assert call(out=O + 4) == -4
    assert call(lat=X + 2) == -4


NO_DEVICE = r"""
import ctypes, math, sys
sys.path.insert(0, %r)
from mla_split_kv_absorbed_amd import _lib as L
from tests.test_abi_cpu import base_args
print(L.lib().mla_decode_partial(ctypes.byref(base_args()), None))
print(L.lib().mla_vup(0x10000, 0x20000000, 0x40000000, 4, 8, 1, None))
print(L.lib().mla_combine_vup(0x10000, 0x400000, 2, 1, 0, None, None, 4, 8, 0x1000000, 1,
                              0x4000000, None, None, None))
# LSE arrays need only their element alignment: these pass validation too
print(L.lib().mla_decode_partial(ctypes.byref(base_args(lse=0x10000 + 0x60000000 + 4)), None))
print(L.lib().mla_combine_vup(0x10000, 0x400002, 2, 1, 1, None, None, 4, 8, 0x1000000, 1,
                              0x4000000, None, None, None))
"""


def test_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    r = subprocess.run([sys.executable, "-c", NO_DEVICE % ROOT], capture_output=True, text=True,
                       timeout=300, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["-7"] * 5, r.stdout + r.stderr


def prologue_base(**over):
    a = L.PrologueArgs()
    a.q_nope, a.q_pe, a.w_uk = FAKE, FAKE + 0x10000000, FAKE + 0x20000000
    a.kv_new, a.positions = FAKE + 0x30000000, FAKE + 0x40000000
    a.dtype = L.MLA_BF16
    a.B, a.S, a.H = 2, 1, 128
    a.rope_theta = 10000.0
    a.kv, a.block_table = FAKE + 0x50000000, FAKE + 0x60000000
    a.block_size, a.max_blocks, a.num_blocks = 32, 4, 8
    a.q_lat, a.q_rope = FAKE + 0x70000000, FAKE + 0x80000000
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(q_nope=None), -1), (dict(q_pe=None), -1), (dict(w_uk=None), -1),
    (dict(kv_new=None), -1), (dict(positions=None), -1), (dict(kv=None), -1),
    (dict(q_lat=None), -1), (dict(q_rope=None), -1), (dict(block_table=None), -1),
    (dict(dtype=9), -3), (dict(B=0), -2), (dict(S=0), -2), (dict(H=0), -2),
    (dict(max_blocks=0), -2), (dict(num_blocks=0), -2),
    (dict(block_size=0), -2),  # contiguous layout takes no block table
    (dict(block_size=0, block_table=None, kv_seq_stride=0), -2),
    (dict(rope_theta=0.0), -4), (dict(rope_theta=float("nan")), -4),
    (dict(rope_theta=float("inf")), -4),
    (dict(q_lat=FAKE + 0x100), -8),           # q_lat overlaps q_nope
    (dict(q_rope=FAKE + 0x50000000), -8),     # q_rope overlaps the cache
    (dict(kv_new=FAKE + 0x50000040), -8),     # the new rows overlap the cache
    (dict(q_pe=FAKE + 0x10000002), -4),       # row tensors 16-byte aligned
    (dict(kv=FAKE + 0x50000008), -4),
])
def test_prologue_validation(over, code):
    a = prologue_base(**over)
    assert L.lib().mla_decode_prologue(ctypes.byref(a), None) == code


def test_noalloc_rejects_before_any_device_call():
    """The allocation-free entry point validates like mla_decode_partial and
    refuses a call whose workspace exceeds its scratch, all on the host."""
    lib = L.lib()
    assert L.mla_noalloc_scratch_bytes() == 96 << 20
    assert lib.mla_decode_partial_noalloc(None, None) == -1
    a = base_args()
    a.q_lat = None
    assert lib.mla_decode_partial_noalloc(ctypes.byref(a), None) == -1
    # 512 heads under the automatic plan: 513 slots x 512 rows x 1028 B > 96 MiB
    a = base_args(H=512)
    need = lib.mla_decode_partial_workspace_size(ctypes.byref(a))
    assert need > 96 << 20
    assert lib.mla_decode_partial_noalloc(ctypes.byref(a), None) == -5


@pytest.mark.parametrize("dtype,stride,flags,path", [
    (L.MLA_BF16, 2, 0, 2), (L.MLA_F16, 8, 0, 2),   # short ranges: the vector kernel
    (L.MLA_BF16, 9, 0, 1), (L.MLA_F16, 64, 0, 1),  # longer: the matrix kernel
    (L.MLA_BF16, 2, L.MLA_FLAG_FORCE_SIMPLE, 0), (L.MLA_F32, 2, 0, 0),
])
def test_contiguous_short_range_routing(dtype, stride, flags, path):
    """A bf16 / fp16 call over a contiguous cache of at most 8 keys per
    sequence takes the short-range kernel (matrix_path 2): it needs no
    workspace and takes no host plan; longer strides keep the matrix kernel."""
    a = base_args(block_size=0, block_table=None, kv_seq_stride=stride, q_dtype=dtype,
                  kv_dtype=dtype, out_dtype=dtype, flags=flags)
    rs = [0] * (a.P * a.B)
    info = L.mla_decode_partial_plan(a, rs, [stride] * (a.P * a.B))
    assert info.matrix_path == path
    assert (L.mla_decode_partial_workspace_size(a) == 0) == (path != 1)
    assert (L.mla_decode_partial_plan_words(a) == 0) == (path != 1)
    if path != 1:
        a.plan, a.plan_chunks = FAKE + 0x48000000, 1
        assert call(a) == -6  # MLA_ERR_UNSUPPORTED


def pair_args(**cur_over):
    """A history call on the matrix kernel and a current-chunk call (2 keys
    per sequence, contiguous) reading the same queries."""
    hist = base_args()
    cur = base_args(block_size=0, block_table=None, kv_seq_stride=2, kv=FAKE + 0x28000000,
                    range_start=FAKE + 0x40002000, range_end=FAKE + 0x40003000, P=1,
                    out=FAKE + 0x58000000, lse=FAKE + 0x68000000, workspace=None,
                    workspace_bytes=0, mask=L.MLA_MASK_CAUSAL_WINDOW)
    for k, v in cur_over.items():
        setattr(cur, k, v)
    return hist, cur


def call_pair(hist, cur):
    return L.lib().mla_decode_partial_pair(ctypes.byref(hist), ctypes.byref(cur), None)


@pytest.mark.parametrize("over,code", [
    (dict(kv_seq_stride=9), -6),                       # current call not short-range
    (dict(flags=L.MLA_FLAG_FORCE_SIMPLE), -6),
    (dict(q_dtype=L.MLA_F16, kv_dtype=L.MLA_F16), -3),  # dtypes differ
    (dict(out=FAKE + 0x10000000), -8),                 # current output over the shared q_rope
    (dict(out=FAKE + 0x50000000 + 256), -8),           # current output over the history output
    (dict(lse=FAKE + 0x70000000 + 64), -8),            # current LSE inside the history workspace
    (dict(kv=None), -1),
])
def test_pair_validation(over, code):
    """Both calls are validated as single calls, then as a pair: the history
    on the matrix kernel, the current call on the short-range kernel, one
    dtype, and no output of either over anything the other touches (the
    shared queries are allowed). Nothing is launched on error."""
    hist, cur = pair_args(**over)
    assert call_pair(hist, cur) == code


def test_pair_valid_call_without_device_reports_hip_error():
    hist, cur = pair_args()
    assert call_pair(hist, cur) == -7
    hist.flags = L.MLA_FLAG_FORCE_SIMPLE
    assert call_pair(hist, cur) == -6


@pytest.mark.parametrize("block_size,path", [(32, 1), (64, 1), (128, 1), (16, 0), (48, 0),
                                             (8, 0), (24, 0), (40, 0)])
def test_paged_block_size_routing(block_size, path):
    """A paged bf16 call takes the matrix kernel when its block size is a
    multiple of the kernel's 32-key tile, else the plain kernel (no
    workspace, no host plan); the plan query reports which."""
    a = base_args(block_size=block_size, max_blocks=256 // block_size + 1)
    n = a.P * a.B
    info = L.mla_decode_partial_plan(a, [0] * n, [200] * n)
    assert info.matrix_path == path
    assert (L.mla_decode_partial_workspace_size(a) == 0) == (path == 0)
    assert (L.mla_decode_partial_plan_words(a) == 0) == (path == 0)
