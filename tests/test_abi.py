"""C ABI checks that need no GPU: the library loads, exports every entry point
include/rib.h declares, and rejects bad arguments before launching anything.

None of these calls reaches a kernel launch: each returns from validation.
"""

import ctypes
import os
import re

import pytest

import windowed_attention_implicit_amd as rib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x7F0000001000)       # aligned, never dereferenced (validation fails first)
MISALIGNED = ctypes.c_void_p(0x7F0000001008)


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "rib.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(rib_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rib.lib_path):
        pytest.fail("librib.so is not built (run __graft_entry__.build())")
    return rib.lib()


def test_exports_every_declared_symbol(L):
    declared = _header_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(L, name), f"{name} declared in rib.h but not exported"
    assert set(declared) == set(rib.exported_symbols)


def test_header_compiles_as_c():
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "rib.h"\nint main(void){ rib_shape_t s = {0}; (void)s; return 0; }\n')
        r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                            "-o", os.path.join(d, "t")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_status_strings(L):
    names = [L.rib_status_string(i).decode() for i in range(5)]
    assert names == ["RIB_OK", "RIB_ERR_INVALID_ARG", "RIB_ERR_UNSUPPORTED", "RIB_ERR_WORKSPACE", "RIB_ERR_HIP"]


def _fwd(L, shape, ws_bytes=1 << 40, ptrs=None, dtype=rib.RIB_BF16, scale=0.0, ws=FAKE):
    p = ptrs or [FAKE] * 6
    return L.rib_window_attn_fwd(ctypes.byref(shape), dtype, scale, p[0], p[1], p[2], p[3], p[4], p[5], None,
                                 ws, ws_bytes, None)


def test_fwd_validation(L):
    good = rib.Shape(2, 192, 192, 6, 32, 96, 16)
    assert _fwd(L, rib.Shape(2, 190, 192, 6, 32, 96, 16)) == rib.RIB_ERR_INVALID_ARG    # H % w
    assert b"multiple" in L.rib_last_error()
    assert _fwd(L, rib.Shape(2, 192, 192, 6, 32, 1, 16)) == rib.RIB_ERR_INVALID_ARG     # w < 2
    assert _fwd(L, rib.Shape(2, 192, 192, 6, 32, 96, 0)) == rib.RIB_ERR_INVALID_ARG     # r < 1
    assert _fwd(L, rib.Shape(-1, 192, 192, 6, 32, 96, 16)) == rib.RIB_ERR_INVALID_ARG   # B < 0
    assert _fwd(L, rib.Shape(2, 192, 192, 6, 48, 96, 16)) == rib.RIB_ERR_UNSUPPORTED    # d_c not 32 or 64
    assert L.rib_fwd_workspace_size(ctypes.byref(rib.Shape(2, 192, 192, 6, 64, 96, 16)), rib.RIB_BF16) > 0
    assert _fwd(L, rib.Shape(2, 192, 192, 6, 32, 96, 33)) == rib.RIB_ERR_UNSUPPORTED    # r > 32
    assert _fwd(L, rib.Shape(1, 512, 512, 1, 32, 512, 16)) == rib.RIB_ERR_UNSUPPORTED   # w > 256
    assert _fwd(L, good, dtype=7) == rib.RIB_ERR_INVALID_ARG
    assert _fwd(L, good, scale=float("nan")) == rib.RIB_ERR_INVALID_ARG
    assert _fwd(L, good, ptrs=[FAKE, None, FAKE, FAKE, FAKE, FAKE]) == rib.RIB_ERR_INVALID_ARG
    assert b"k_c" in L.rib_last_error()
    assert _fwd(L, good, ptrs=[FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE]) == rib.RIB_ERR_INVALID_ARG
    assert b"aligned" in L.rib_last_error()
    need = L.rib_fwd_workspace_size(ctypes.byref(good), rib.RIB_BF16)
    assert need > 0
    assert _fwd(L, good, ws_bytes=need - 1) == rib.RIB_ERR_WORKSPACE
    assert _fwd(L, good, ws=None) == rib.RIB_ERR_WORKSPACE
    assert _fwd(L, good, ws=MISALIGNED) == rib.RIB_ERR_INVALID_ARG
    # an empty batch is a valid no-op
    assert _fwd(L, rib.Shape(0, 192, 192, 6, 32, 96, 16), ptrs=[None] * 6, ws=None, ws_bytes=0) == rib.RIB_OK


def test_fwd_noalloc_validation(L):
    """The allocation-free forward: argument errors as for the forward, shapes whose workspace
    exceeds the library's per-GPU array rejected before any device call, empty batches valid."""
    def call(shape, ptrs=None, dtype=rib.RIB_BF16):
        p = ptrs or [FAKE] * 6
        return L.rib_window_attn_fwd_noalloc(ctypes.byref(shape), dtype, 0.0, p[0], p[1], p[2], p[3], p[4], p[5],
                                             None, None)
    assert call(rib.Shape(2, 190, 192, 6, 32, 32, 16)) == rib.RIB_ERR_INVALID_ARG
    assert call(rib.Shape(2, 192, 192, 6, 32, 32, 16), ptrs=[FAKE, None, FAKE, FAKE, FAKE, FAKE]) == \
        rib.RIB_ERR_INVALID_ARG
    assert call(rib.Shape(2, 192, 192, 6, 32, 32, 16), ptrs=[FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE]) == \
        rib.RIB_ERR_INVALID_ARG
    # the 96x96 workload needs about 150 MB of workspace: more than the array holds
    big = rib.Shape(4, 192, 192, 6, 32, 96, 16)
    assert L.rib_fwd_workspace_size(ctypes.byref(big), rib.RIB_BF16) > rib.NOALLOC_WORKSPACE_BYTES
    assert call(big) == rib.RIB_ERR_WORKSPACE
    assert b"allocation-free" in L.rib_last_error()
    # the small-window layers of a [2, 192, 192, 6, 32] map fit
    for w in (16, 32):
        s = rib.Shape(2, 192, 192, 6, 32, w, 16)
        assert 0 < L.rib_fwd_workspace_size(ctypes.byref(s), rib.RIB_BF16) <= rib.NOALLOC_WORKSPACE_BYTES
    assert call(rib.Shape(0, 192, 192, 6, 32, 32, 16)) == rib.RIB_OK


def test_rpb_validation(L):
    good = rib.Shape(2, 192, 192, 6, 32, 96, 0)     # r is ignored by the RPB kernel

    def call(shape, ws_bytes=1 << 40, dtype=rib.RIB_BF16, nulls=(), ws=FAKE, table=FAKE):
        p = [None if i in nulls else FAKE for i in range(3)]
        return L.rib_rpb_window_attn_fwd(ctypes.byref(shape), dtype, 0.0, *p, table, FAKE, None, ws, ws_bytes,
                                         None)

    need = L.rib_rpb_fwd_workspace_size(ctypes.byref(good), rib.RIB_BF16)
    # K and V^T windowed copies, the fp16 tables and per-key offsets: linear, no N x N bias
    assert 2 * 2 * 192 * 192 * 6 * 32 * 2 <= need <= 2 * 2 * 192 * 192 * 6 * 32 * 2 + (1 << 20)
    assert call(good, dtype=rib.RIB_F32) == rib.RIB_ERR_UNSUPPORTED
    assert b"bfloat16" in L.rib_last_error()
    assert L.rib_rpb_fwd_workspace_size(ctypes.byref(good), rib.RIB_F32) == 0
    assert call(rib.Shape(1, 122, 122, 1, 32, 122, 0)) == rib.RIB_ERR_UNSUPPORTED      # table too large for LDS
    assert b"LDS" in L.rib_last_error()
    assert call(rib.Shape(1, 121, 121, 1, 32, 121, 0), ws=None) == rib.RIB_ERR_WORKSPACE   # w = 121 fits
    assert call(rib.Shape(2, 192, 192, 6, 64, 96, 0)) == rib.RIB_ERR_UNSUPPORTED        # d_c
    assert call(rib.Shape(2, 190, 192, 6, 32, 96, 0)) == rib.RIB_ERR_INVALID_ARG        # H % w
    assert call(good, table=None) == rib.RIB_ERR_INVALID_ARG
    assert b"table" in L.rib_last_error()
    assert call(good, nulls=(1,)) == rib.RIB_ERR_INVALID_ARG
    assert call(good, ws_bytes=need - 1) == rib.RIB_ERR_WORKSPACE
    assert call(good, ws=MISALIGNED, ws_bytes=need) == rib.RIB_ERR_INVALID_ARG
    assert call(rib.Shape(0, 192, 192, 6, 32, 96, 0), nulls=(0, 1, 2), ws=None, ws_bytes=0, table=None) == rib.RIB_OK


def test_cla_validation(L):
    good = rib.Shape(2, 192, 192, 6, 32, 96, 16)

    def gate(shape, dtype=rib.RIB_BF16, x=FAKE, w_dw=FAKE, w_pw=FAKE, g=FAKE):
        return L.rib_cla_gate(ctypes.byref(shape), dtype, x, w_dw, None, w_pw, None, g, None)

    assert gate(rib.Shape(1, 8, 8, 9, 32, 2, 1)) == rib.RIB_ERR_UNSUPPORTED      # C = 288 > 256
    assert b"multiples of 32" in L.rib_last_error()
    assert gate(rib.Shape(1, 8, 8, 3, 16, 2, 1)) == rib.RIB_ERR_UNSUPPORTED      # C = 48
    assert gate(rib.Shape(1, 0, 8, 2, 32, 2, 1)) == rib.RIB_ERR_INVALID_ARG
    assert gate(good, dtype=5) == rib.RIB_ERR_INVALID_ARG
    assert gate(good, w_dw=None) == rib.RIB_ERR_INVALID_ARG
    assert gate(good, g=MISALIGNED) == rib.RIB_ERR_INVALID_ARG
    assert gate(rib.Shape(0, 8, 8, 2, 32, 2, 1), x=None, g=None) == rib.RIB_OK
    # the gated forward validates like the plain forward and requires the gate
    need = L.rib_fwd_workspace_size(ctypes.byref(good), rib.RIB_BF16)
    args = [FAKE] * 5
    assert L.rib_window_attn_fwd_gated(ctypes.byref(good), rib.RIB_BF16, 0.0, *args, None, FAKE, None, FAKE, need,
                                       None) == rib.RIB_ERR_INVALID_ARG
    assert b"gate" in L.rib_last_error()
    assert L.rib_window_attn_fwd_gated(ctypes.byref(good), rib.RIB_BF16, 0.0, *args, MISALIGNED, FAKE, None, FAKE,
                                       need, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_window_attn_fwd_gated(ctypes.byref(good), rib.RIB_BF16, 0.0, *args, FAKE, FAKE, None, FAKE,
                                       need - 1, None) == rib.RIB_ERR_WORKSPACE


def test_bwd_validation(L):
    good = rib.Shape(2, 192, 192, 6, 32, 64, 16)
    need = L.rib_bwd_workspace_size(ctypes.byref(good), rib.RIB_BF16)
    assert need > 0

    def call(shape, ws_bytes, nulls=()):
        p = [None if i in nulls else FAKE for i in range(13)]
        return L.rib_window_attn_bwd(ctypes.byref(shape), rib.RIB_BF16, 0.0, *p, FAKE, ws_bytes, None)

    assert call(rib.Shape(2, 192, 100, 6, 32, 64, 16), need) == rib.RIB_ERR_INVALID_ARG
    assert call(good, need, nulls=(6,)) == rib.RIB_ERR_INVALID_ARG        # lse is required
    assert b"lse" in L.rib_last_error()
    assert call(good, need, nulls=(12,)) == rib.RIB_ERR_INVALID_ARG       # dk_p
    assert call(good, need - 256) == rib.RIB_ERR_WORKSPACE


def test_posgen_validation(L):
    mlp = rib._Mlp(16, 64, 16, FAKE.value, None, FAKE.value, None)
    assert L.rib_posgen(1, ctypes.byref(mlp), rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_posgen(96, None, rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_INVALID_ARG
    bad = rib._Mlp(16, 64, 33, FAKE.value, None, FAKE.value, None)
    assert L.rib_posgen(96, ctypes.byref(bad), rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_UNSUPPORTED
    bad = rib._Mlp(17, 64, 16, FAKE.value, None, FAKE.value, None)
    assert L.rib_posgen(96, ctypes.byref(bad), rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_posgen(96, ctypes.byref(mlp), rib.RIB_BF16, None, FAKE, None) == rib.RIB_ERR_INVALID_ARG


def test_posgen_bwd_validation(L):
    """Every call below fails validation before any launch (FAKE is never dereferenced)."""
    mlp = rib._Mlp(16, 64, 16, FAKE.value, None, FAKE.value, None)
    need = L.rib_posgen_bwd_workspace_size(96, ctypes.byref(mlp))
    # one partial set per block: min(tiles, 1024) blocks, tiles of 32 tokens at w = 96 ...
    assert need == 4 * (96 * 96 // 32) * (64 * 64 + 64 + 32 * 64 + 32)
    # ... and of a single token when 25 tokens could not otherwise make 128 tiles
    small = rib._Mlp(4, 8, 2, FAKE.value, None, FAKE.value, None)
    assert L.rib_posgen_bwd_workspace_size(5, ctypes.byref(small)) == 4 * 25 * (8 * 16 + 8 + 4 * 8 + 4)
    assert L.rib_posgen_bwd_workspace_size(1, ctypes.byref(mlp)) == 0
    assert L.rib_posgen_bwd_workspace_size(96, None) == 0

    def call(w=96, m=mlp, dq=FAKE, dk=FAKE, dw1=FAKE, db1=FAKE, dw2=FAKE, db2=FAKE, ws=FAKE, nbytes=None):
        return L.rib_posgen_bwd(w, None if m is None else ctypes.byref(m), dq, dk, dw1, db1, dw2, db2, ws,
                                need if nbytes is None else nbytes, None)

    assert call(w=1) == rib.RIB_ERR_INVALID_ARG
    assert call(w=257) == rib.RIB_ERR_UNSUPPORTED
    assert call(m=None) == rib.RIB_ERR_INVALID_ARG
    assert call(m=rib._Mlp(16, 64, 33, FAKE.value, None, FAKE.value, None)) == rib.RIB_ERR_UNSUPPORTED
    big = rib._Mlp(16, 128, 32, FAKE.value, None, FAKE.value, None)   # the weights alone exceed 64 KB
    assert call(m=big) == rib.RIB_ERR_UNSUPPORTED
    assert call(m=rib._Mlp(16, 64, 16, None, None, FAKE.value, None)) == rib.RIB_ERR_INVALID_ARG
    assert call(dq=None) == rib.RIB_ERR_INVALID_ARG
    assert call(dk=None) == rib.RIB_ERR_INVALID_ARG
    assert call(dw1=None) == rib.RIB_ERR_INVALID_ARG
    assert call(dw2=None) == rib.RIB_ERR_INVALID_ARG
    assert call(dq=ctypes.c_void_p(FAKE.value + 2)) == rib.RIB_ERR_INVALID_ARG
    assert call(ws=None) == rib.RIB_ERR_WORKSPACE
    assert call(nbytes=need - 4) == rib.RIB_ERR_WORKSPACE


def test_partition_validation(L):
    s = rib.Shape(1, 96, 96, 6, 32, 96, 1)
    assert L.rib_window_partition(ctypes.byref(s), rib.RIB_BF16, None, FAKE, None) == rib.RIB_ERR_INVALID_ARG
    s2 = rib.Shape(1, 96, 90, 6, 32, 96, 1)
    assert L.rib_window_unpartition(ctypes.byref(s2), rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_INVALID_ARG
    s3 = rib.Shape(1, 96, 96, 6, 4, 96, 1)   # 4 bf16 channels = 8 bytes per row
    assert L.rib_window_partition(ctypes.byref(s3), rib.RIB_BF16, FAKE, FAKE, None) == rib.RIB_ERR_UNSUPPORTED


def test_workspace_is_linear_not_quadratic(L):
    """No N x N buffer: the workspace grows with the map, not with the window area squared."""
    def ws(B, H, w, fn=L.rib_fwd_workspace_size):
        return fn(ctypes.byref(rib.Shape(B, H, H, 6, 32, w, 16)), rib.RIB_BF16)
    # the bf16 forward's split-tail pieces (w*w >= 2048): a fixed cap of 1024 pieces of
    # 256 queries x (32 + 2) floats, independent of the map and the window
    # windows whose side divides 64 read K_c and V in their maps: almost no forward workspace
    assert ws(2, 192, 16) <= 1 << 20 and ws(2, 192, 32) <= 1 << 20
    # ... and the backward's gather writes no K_c, V rows for them: two windowed copies fewer
    bw = L.rib_bwd_workspace_size
    copy = 2 * 192 * 192 * 6 * 32 * 2
    assert ws(2, 192, 16, bw) <= ws(2, 192, 24, bw) - 2 * copy + (1 << 20)
    for fn, split_cap, w_small in ((L.rib_fwd_workspace_size, 1024 * 256 * 34 * 4, 24),
                                   (L.rib_bwd_workspace_size, 0, 24)):
        small, big = ws(2, 192, w_small, fn), ws(2, 192, 96, fn)
        # same map, 36x larger windows: only the per-window-size parts (positional tokens, their
        # transposes and per-unit partials, a few MB at w = 96) differ
        assert abs(big - small) <= 0.03 * small + (4 << 20) + split_cap
        assert ws(4, 192, 96, fn) <= 2 * ws(2, 192, 96, fn) + 4096
        N = 96 * 96
        assert big < 2 * 6 * N * N                          # far below one N x N matrix per unit
    assert L.rib_fwd_workspace_size(ctypes.byref(rib.Shape(1, 10, 10, 1, 32, 3, 16)), rib.RIB_BF16) == 0


def test_timing_select(L):
    """Group masks: any subset of the groups is accepted, a bit past the last group is rejected and
    leaves the previous selection; no events are recorded without a call."""
    n = len(rib.KERNEL_GROUPS)
    assert L.rib_kernel_timing_select(1 << rib.KERNEL_GROUPS["attn_fwd"]) == rib.RIB_OK
    assert L.rib_kernel_timing_select((1 << n) - 1) == rib.RIB_OK
    assert L.rib_kernel_timing_select(1 << n) == rib.RIB_ERR_INVALID_ARG
    assert b"past the last" in L.rib_last_error()
    assert L.rib_kernel_timing_select(0) == rib.RIB_OK
    assert L.rib_kernel_timing_enable(1) == rib.RIB_OK and L.rib_kernel_timing_enable(0) == rib.RIB_OK
    rib.kernel_timing_select("attn_fwd", "posgen")
    rib.kernel_timing_select()
