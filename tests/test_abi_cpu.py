"""The C ABI on a host without a GPU: exports, validation, workspace sizing.

Every call here fails validation (or the device check) before anything is
enqueued, so no pointer is ever dereferenced.  Tests that rely on the device
check failing are skipped where a GPU is present.
"""
import ctypes
import os
import re

import pytest
import torch

import mlp_prefill_amd as m
from mlp_prefill_amd import nvfp4_tensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")

FAKE = 0x100000          # aligned, never dereferenced


def _t(c=FAKE, s=FAKE, g=FAKE):
    return nvfp4_tensor(c, s, g)


def _size():
    return ctypes.c_size_t(0)


def test_library_exports_every_declared_function():
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nvfp4_\w+)\s*\(", text, re.M))
    assert {"nvfp4_quantize_act", "nvfp4_gemm", "nvfp4_mlp_gu_act", "nvfp4_mlp_down",
            "nvfp4_grouped_gemm", "nvfp4_strerror", "nvfp4_launch_count"} <= names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    # and nothing else: the library is built with hidden visibility
    import subprocess
    nm = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = {ln.split()[-1] for ln in nm.stdout.splitlines() if " T " in ln}
        assert exported == names, sorted(exported ^ names)


def test_strerror_covers_all_codes():
    for code in range(8):
        assert m.lib.nvfp4_strerror(code)
    assert m.lib.nvfp4_strerror(99) == b"unknown status"


def test_quantize_validation():
    q = m.lib.nvfp4_quantize_act
    sz = ctypes.c_size_t(1 << 20)
    assert q(FAKE, 7, 4, 32, 32, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_ARG        # dtype
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), 9, FAKE, ctypes.byref(sz), None) == m.ERR_ARG   # gs mode
    assert q(FAKE, m.BF16, 4, 24, 24, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_SHAPE  # cols % 16
    assert q(FAKE, m.BF16, 4, 32, 16, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_SHAPE  # ld < cols
    assert q(FAKE, m.BF16, -1, 32, 32, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_SHAPE
    assert q(None, m.BF16, 4, 32, 32, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_NULL
    assert q(FAKE, m.BF16, 4, 32, 32, _t(g=0), 0, FAKE, ctypes.byref(sz), None) == m.ERR_NULL
    assert q(FAKE + 2, m.BF16, 4, 32, 32, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_ALIGN
    assert q(FAKE, m.BF16, 4, 32, 36, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_ALIGN   # row stride
    assert q(FAKE, m.BF16, 4, 32, 32, _t(c=FAKE + 8), 0, FAKE, ctypes.byref(sz), None) == m.ERR_ALIGN
    small = ctypes.c_size_t(16)
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), 0, FAKE, ctypes.byref(small), None) == m.ERR_WORKSPACE
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), 0, FAKE, None, None) == m.ERR_WORKSPACE
    # zero rows: a successful no-op even with NULL data pointers
    assert q(None, m.BF16, 0, 32, 32, nvfp4_tensor(0, 0, 0), 0, FAKE, ctypes.byref(sz), None) == m.OK
    # NVFP4_GS_FROM_AMAX: ws holds the AMAX_SLOTS partial maxima (float32, 16-byte aligned)
    slots = ctypes.c_size_t(4 * m.AMAX_SLOTS)
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), m.GS_FROM_AMAX, None, None, None) == m.ERR_WORKSPACE
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), m.GS_FROM_AMAX, FAKE, ctypes.byref(ctypes.c_size_t(4)), None) \
        == m.ERR_WORKSPACE
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), m.GS_FROM_AMAX, FAKE + 4, ctypes.byref(slots), None) == m.ERR_ALIGN
    s = _size()
    assert q(None, m.BF16, 4, 32, 32, nvfp4_tensor(0, 0, 0), m.GS_FROM_AMAX, None, ctypes.byref(s), None) == m.OK
    assert s.value == 4 * m.AMAX_SLOTS
    assert m.lib.nvfp4_quantize_act_noalloc(FAKE, m.BF16, 4, 32, 32, _t(), m.GS_FROM_AMAX, None) == m.ERR_ARG


def test_quantize_noalloc_validation():
    q = m.lib.nvfp4_quantize_act_noalloc
    assert q(FAKE, 7, 4, 32, 32, _t(), 0, None) == m.ERR_ARG                  # dtype
    assert q(FAKE, m.BF16, 4, 32, 32, _t(), 9, None) == m.ERR_ARG             # gs mode
    assert q(FAKE, m.BF16, 4, 24, 24, _t(), 0, None) == m.ERR_SHAPE           # cols % 16
    assert q(FAKE, m.BF16, 4, 32, 16, _t(), 0, None) == m.ERR_SHAPE           # ld < cols
    assert q(FAKE, m.BF16, 1 << 28, 256, 256, _t(), 0, None) == m.ERR_SHAPE   # 2^32 blocks
    assert q(None, m.BF16, 4, 32, 32, _t(), 0, None) == m.ERR_NULL
    assert q(FAKE, m.BF16, 4, 32, 32, _t(s=0), 0, None) == m.ERR_NULL
    assert q(FAKE + 2, m.BF16, 4, 32, 32, _t(), 0, None) == m.ERR_ALIGN
    assert q(FAKE, m.BF16, 4, 32, 36, _t(), 0, None) == m.ERR_ALIGN           # row stride
    assert q(None, m.BF16, 0, 32, 32, nvfp4_tensor(0, 0, 0), 0, None) == m.OK  # empty: no-op


@no_gpu
def test_quantize_noalloc_without_device():
    assert m.lib.nvfp4_quantize_act_noalloc(FAKE, m.BF16, 4, 32, 32, _t(), 0, None) == m.ERR_DEVICE


def test_whole_mlp_validation_and_workspace():
    f = m.lib.nvfp4_mlp
    z = nvfp4_tensor(0, 0, 0)
    big = ctypes.c_size_t(1 << 30)
    t = _t()

    def call(x=FAKE, xdt=m.BF16, ldx=5120, xa=None, T=4, K=5120, I=17408, wg=t, y=FAKE, ydt=m.F32, ldy=5120,
             ya=None, ws=FAKE, sz=None):
        return f(x, xdt, ldx, xa, T, K, I, wg, t, t, t, t, y, ydt, ldy, ya, ws,
                 ctypes.byref(big if sz is None else sz), None)
    assert call(xdt=5) == m.ERR_ARG
    assert call(ydt=7) == m.ERR_ARG
    assert call(K=5000, ldx=5000, ldy=5000) == m.ERR_SHAPE          # K % 128
    assert call(I=17400) == m.ERR_SHAPE                              # I % 128
    assert call(ldx=5000) == m.ERR_SHAPE                             # ld_x < K
    assert call(ldy=4096) == m.ERR_SHAPE                             # ldy < K
    assert call(T=-1) == m.ERR_SHAPE
    assert call(x=None) == m.ERR_NULL
    assert call(y=None) == m.ERR_NULL
    assert call(wg=_t(g=0)) == m.ERR_NULL
    assert call(x=FAKE + 8) == m.ERR_ALIGN
    assert call(xa=FAKE + 4) == m.ERR_ALIGN                          # x_amax
    assert call(ya=FAKE + 4) == m.ERR_ALIGN                          # y_amax
    assert call(sz=ctypes.c_size_t(64)) == m.ERR_WORKSPACE
    assert call(xa=FAKE, ya=FAKE) == m.ERR_ARG                       # x_amax and y_amax alias
    assert f(None, m.BF16, 5120, None, 0, 5120, 17408, z, z, z, z, z, None, m.F32, 5120, None, None, None,
             None) == m.OK                                           # T = 0: no-op
    # workspace: decode path [H][partials][down partial sums][tickets][gate/up partial sums];
    # large batches: the separate calls' sum
    s = _size()
    assert f(None, m.BF16, 5120, None, 1, 5120, 17408, z, z, z, z, z, None, m.F32, 5120, None, None,
             ctypes.byref(s), None) == m.OK
    # T = 1: the down projection's K = 17408 runs in 9 splits (8 of two 1024-wide units + 1)
    assert s.value == 17408 * 4 + 17408 // 4 * 4 + 9 * 5120 * 4 + 5120 // 4 * 4
    # T = 5 (16x16x32 stream, splits of 8 stages of 256): down 9 splits, gate/up 3 splits
    # with its partial sums [3][5][2 x 17408] and 1088 tickets after the 160 of the down
    assert f(None, m.BF16, 5120, None, 5, 5120, 17408, z, z, z, z, z, None, m.F32, 5120, None, None,
             ctypes.byref(s), None) == m.OK
    assert s.value == 5 * 17408 * 4 + 1088 * 4 + 9 * 5 * 5120 * 4 + 5120 + 3 * 5 * 2 * 17408 * 4
    assert f(None, m.BF16, 5120, None, 1024, 5120, 17408, z, z, z, z, z, None, m.F32, 5120, None, None,
             ctypes.byref(s), None) == m.OK
    assert s.value >= m.mlp_gu_act_ws_bytes(1024, 5120, 17408) + m.mlp_down_ws_bytes(1024, 17408, 5120)


@no_gpu
def test_whole_mlp_without_device():
    t = _t()
    big = ctypes.c_size_t(1 << 30)
    assert m.lib.nvfp4_mlp(FAKE, m.BF16, 5120, None, 1, 5120, 17408, t, t, t, t, t, FAKE, m.F32, 5120, None, FAKE,
                           ctypes.byref(big), None) == m.ERR_DEVICE


def test_quantize_workspace_query():
    q = m.lib.nvfp4_quantize_act
    s = _size()
    assert q(None, m.BF16, 1024, 5120, 5120, nvfp4_tensor(0, 0, 0), m.GS_COMPUTE, None, ctypes.byref(s), None) == m.OK
    assert 0 < s.value <= 16384
    s = _size()
    assert q(None, m.BF16, 1024, 5120, 5120, nvfp4_tensor(0, 0, 0), m.GS_GIVEN, None, ctypes.byref(s), None) == m.OK
    assert s.value == 0


def test_gemm_and_down_validation():
    g = m.lib.nvfp4_gemm
    big = ctypes.c_size_t(1 << 30)
    ws = (FAKE, ctypes.byref(big), None)
    assert g(_t(), _t(), 4, 8, 100, FAKE, m.F32, 8, None, *ws) == m.ERR_SHAPE        # K % 128
    assert g(_t(), _t(), 4, 8, 128, FAKE, 5, 8, None, *ws) == m.ERR_ARG
    assert g(_t(), _t(), 4, 8, 128, FAKE, m.F32, 4, None, *ws) == m.ERR_SHAPE        # ldc < N
    assert g(_t(), _t(), 4, 8, 128, None, m.F32, 8, None, *ws) == m.ERR_NULL
    assert g(_t(), _t(), 4, 6, 128, FAKE, m.F32, 6, None, *ws) == m.ERR_ALIGN        # row stride 24 B
    assert g(_t(), _t(s=FAKE + 4), 4, 8, 128, FAKE, m.F32, 8, None, *ws) == m.ERR_ALIGN
    assert g(_t(), _t(), 4, 8, 128, FAKE, m.F32, 8, None, None, None, None) == m.ERR_WORKSPACE
    assert g(_t(), _t(), 0, 8, 128, None, m.F32, 8, None, None, None, None) == m.OK   # empty
    s = _size()
    assert g(nvfp4_tensor(0, 0, 0), nvfp4_tensor(0, 0, 0), 1024, 5120, 17408, None, m.F32, 5120, None, None,
             ctypes.byref(s), None) == m.OK
    # f16 activation copy + float32 partials of the 4 K splits: 1024 tokens in
    # 64 x 256 tiles make 16 x 20 = 320 work-groups, split 4 ways to 1280
    assert s.value == 1024 * 17408 * 2 + 4 * 1024 * 5120 * 4
    assert g(nvfp4_tensor(0, 0, 0), nvfp4_tensor(0, 0, 0), 4096, 4096, 4096, None, m.F32, 4096, None, None,
             ctypes.byref(s), None) == m.OK
    assert s.value == 4096 * 4096 * 2 + 4096 * 4096 * 4   # 64 x 16 = 1024 tiles: one split
    assert g(_t(), _t(), 4, 8, 128, FAKE, m.F32, 8, FAKE + 4, *ws) == m.ERR_ALIGN  # c_amax
    d = m.lib.nvfp4_mlp_down
    assert d(_t(), _t(), 4, 128, 64, FAKE, m.F32, 64, FAKE + 8, *ws) == m.ERR_ALIGN  # y_amax
    assert d(_t(), _t(), 4, 100, 64, FAKE, m.F32, 64, None, *ws) == m.ERR_SHAPE      # I % 128
    assert d(_t(), _t(), 4, 128, 64, FAKE, m.BF16, 60, None, *ws) == m.ERR_SHAPE     # ldy < K
    assert d(_t(), _t(), 4, 128, 64, None, m.F32, 64, None, *ws) == m.ERR_NULL


def test_tile_weight_validation_and_size():
    tw = m.lib.nvfp4_tile_weight
    s = _size()
    # 128-row groups x 128-K chunks x 9216 bytes (8 KiB codes + 1 KiB scales)
    assert tw(nvfp4_tensor(0, 0, 0), 1, 17408, 5120, None, ctypes.byref(s), None) == m.OK
    assert s.value == 136 * 40 * 9216
    assert tw(nvfp4_tensor(0, 0, 0), 64, 2048, 4096, None, ctypes.byref(s), None) == m.OK
    assert s.value == 64 * 16 * 32 * 9216
    assert tw(nvfp4_tensor(0, 0, 0), 1, 200, 256, None, ctypes.byref(s), None) == m.OK
    assert s.value == 2 * 2 * 9216                                   # the last group of 128 rows is partial
    assert m.tile_weight_bytes(5120, 17408) == 40 * 136 * 9216
    big = ctypes.c_size_t(1 << 30)
    assert tw(_t(), 1, 64, 100, FAKE, ctypes.byref(big), None) == m.ERR_SHAPE    # K % 128
    assert tw(_t(), 1, -1, 128, FAKE, ctypes.byref(big), None) == m.ERR_SHAPE
    assert tw(_t(), 0, 64, 128, FAKE, ctypes.byref(big), None) == m.ERR_ARG      # experts
    assert tw(_t(), 1, 65536, 65536, FAKE, ctypes.byref(big), None) == m.ERR_SHAPE   # one expert's copy >= 2 GiB
    assert tw(_t(), 1, 64, 128, FAKE + 16, ctypes.byref(big), None) == m.ERR_ALIGN
    assert tw(_t(c=0), 1, 64, 128, FAKE, ctypes.byref(big), None) == m.ERR_NULL
    assert tw(_t(s=FAKE + 4), 1, 64, 128, FAKE, ctypes.byref(big), None) == m.ERR_ALIGN
    small = ctypes.c_size_t(9215)
    assert tw(_t(), 1, 64, 128, FAKE, ctypes.byref(small), None) == m.ERR_WORKSPACE
    assert tw(_t(), 1, 0, 128, None, None, None) == m.OK                          # empty: no-op
    # a weight operand's tiled copy must be 256-byte aligned
    ws = (FAKE, ctypes.byref(big), None)
    wt = nvfp4_tensor(FAKE, FAKE, FAKE, FAKE + 64)
    assert m.lib.nvfp4_gemm(_t(), wt, 4, 8, 128, FAKE, m.F32, 8, None, *ws) == m.ERR_ALIGN


@no_gpu
def test_tile_weight_without_device():
    big = ctypes.c_size_t(1 << 30)
    before = m.lib.nvfp4_launch_count()
    assert m.lib.nvfp4_tile_weight(_t(), 1, 64, 128, FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_launch_count() == before


@pytest.mark.parametrize("name", ["nvfp4_moe_mlp", "nvfp4_moe_mlp_static"])
def test_moe_mlp_validation_and_workspace(name):
    f = getattr(m.lib, name)
    static = name.endswith("static")
    big = ctypes.c_size_t(1 << 34)
    t3 = (_t(), _t(), _t(), _t(), _t())

    def call(x=FAKE, xd=m.BF16, ldx=256, t=96, k=256, i=384, e=8, rows=FAKE, offs=FAKE, mm=192, y=FAKE, yd=m.F32,
             ldy=256, ws=FAKE, sz=None, tens=t3):
        return f(x, xd, ldx, t, k, i, e, rows, offs, mm, *tens, y, yd, ldy, ws, ctypes.byref(sz or big), None)

    assert call(xd=7) == m.ERR_ARG
    assert call(yd=7) == m.ERR_ARG
    assert call(e=0) == m.ERR_ARG
    assert call(k=200, ldx=200, ldy=200) == m.ERR_SHAPE          # K % 128
    assert call(i=200) == m.ERR_SHAPE                            # I % 128
    assert call(ldx=128) == m.ERR_SHAPE                          # ld_x < K
    assert call(ldy=128) == m.ERR_SHAPE
    assert call(t=1 << 22, k=1024, ldx=1024, ldy=1024) == m.ERR_SHAPE   # T * K * 2 >= 2^31
    assert call(rows=None) == m.ERR_NULL
    assert call(y=None) == m.ERR_NULL
    assert call(rows=FAKE + 2) == m.ERR_ALIGN
    assert call(y=FAKE + 8) == m.ERR_ALIGN
    assert call(tens=(_t(), _t(s=FAKE + 4), _t(), _t(), _t())) == m.ERR_ALIGN
    assert call(sz=ctypes.c_size_t(256)) == m.ERR_WORKSPACE
    assert f(None, m.BF16, 256, 0, 256, 384, 8, None, None, 0, *t3, None, m.F32, 256, None, None, None) == m.OK
    s = _size()
    assert f(None, m.BF16, 4096, 4096, 4096, 2048, 64, None, None, 32768, *(nvfp4_tensor(0, 0, 0),) * 5, None, m.BF16,
             4096, None, ctypes.byref(s), None) == m.OK
    # x f16 copy + float32 H (not with static scales: the gate/up quantises H itself) + f16 H~ + the down
    # projection's partial sums: no gathered activation copy
    h32 = 0 if static else 32768 * 2048 * 4
    assert s.value >= 4096 * 4096 * 2 + h32 + 32768 * 2048 * 2
    assert s.value < 4096 * 4096 * 2 + h32 + 32768 * 2048 * 2 + 32768 * 4096 * 4 + (1 << 24)
    assert m.moe_mlp_ws_bytes(4096, 4096, 2048, 64, 32768, static=static) == s.value


@no_gpu
@pytest.mark.parametrize("name", ["nvfp4_moe_mlp", "nvfp4_moe_mlp_static"])
def test_moe_mlp_without_device(name):
    big = ctypes.c_size_t(1 << 34)
    before = m.lib.nvfp4_launch_count()
    assert getattr(m.lib, name)(FAKE, m.BF16, 256, 96, 256, 384, 8, FAKE, FAKE, 192, _t(), _t(), _t(), _t(), _t(),
                                FAKE, m.F32, 256, FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_launch_count() == before


def test_gu_act_validation_and_workspace():
    f = m.lib.nvfp4_mlp_gu_act
    z = nvfp4_tensor(0, 0, 0)
    s = _size()
    assert f(z, z, z, 1024, 5120, 17408, z, None, ctypes.byref(s), None) == m.OK
    assert s.value >= 1024 * 17408 * 4
    assert f(z, z, z, 4, 5120, 17400, z, None, ctypes.byref(s), None) == m.ERR_SHAPE
    small = ctypes.c_size_t(1024)
    assert f(_t(), _t(), _t(), 4, 128, 128, _t(), FAKE, ctypes.byref(small), None) == m.ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 24)
    assert f(_t(), _t(), _t(), 4, 128, 128, _t(), FAKE + 64, ctypes.byref(big), None) == m.ERR_ALIGN
    assert f(_t(), _t(c=0), _t(), 4, 128, 128, _t(), FAKE, ctypes.byref(big), None) == m.ERR_NULL
    assert f(z, z, z, 0, 128, 128, z, FAKE, ctypes.byref(big), None) == m.OK


def test_static_scale_entry_points_validation_and_workspace():
    f = m.lib.nvfp4_mlp_gu_act_static
    z = nvfp4_tensor(0, 0, 0)
    s = _size()
    assert f(z, z, z, 1024, 5120, 17408, z, None, ctypes.byref(s), None) == m.OK
    assert s.value == 1024 * 5120 * 2                     # only the f16 copy of x~: no float32 H
    assert f(z, z, z, 4, 5120, 17400, z, None, ctypes.byref(s), None) == m.ERR_SHAPE
    small = ctypes.c_size_t(1024)
    assert f(_t(), _t(), _t(), 64, 128, 128, _t(), FAKE, ctypes.byref(small), None) == m.ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 24)
    assert f(_t(), _t(), _t(), 4, 128, 128, _t(g=0), FAKE, ctypes.byref(big), None) == m.ERR_NULL   # gscale read
    assert f(_t(), _t(), _t(), 4, 128, 128, _t(s=FAKE + 4), FAKE, ctypes.byref(big), None) == m.ERR_ALIGN
    assert f(z, z, z, 0, 128, 128, z, FAKE, ctypes.byref(big), None) == m.OK
    d = m.lib.nvfp4_mlp_down_quant
    assert d(z, z, 1024, 17408, 5120, z, None, ctypes.byref(s), None) == m.OK
    s2 = _size()
    assert m.lib.nvfp4_mlp_down(z, z, 1024, 17408, 5120, None, m.F32, 5120, None, None, ctypes.byref(s2), None) == m.OK
    assert s.value == s2.value                            # same split plan as the float32 down projection
    assert d(_t(), _t(), 4, 100, 64, _t(), FAKE, ctypes.byref(big), None) == m.ERR_SHAPE      # I % 128
    assert d(_t(), _t(), 4, 128, 40, _t(), FAKE, ctypes.byref(big), None) == m.ERR_SHAPE      # K % 16
    assert d(_t(), _t(), 4, 128, 64, _t(c=0), FAKE, ctypes.byref(big), None) == m.ERR_NULL
    assert d(_t(), _t(), 0, 128, 64, z, FAKE, ctypes.byref(big), None) == m.OK


def test_grouped_validation():
    f = m.lib.nvfp4_grouped_gemm
    sz = ctypes.c_size_t(1 << 30)
    args = lambda **kw: dict(dict(a=_t(), rows=FAKE, off=FAKE, E=4, M=64, w0=_t(), w1=_t(), N=128, K=128,
                                  epi=m.EPI_STORE, out=FAKE, dt=m.F32, ld=128, oq=_t()), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["a"], a["rows"], a["off"], a["E"], a["M"], a["w0"], a["w1"], a["N"], a["K"], a["epi"],
                 a["out"], a["dt"], a["ld"], a["oq"], FAKE, ctypes.byref(sz), None)
    assert call(E=0) == m.ERR_ARG
    assert call(epi=5) == m.ERR_ARG
    assert call(epi=m.EPI_SILU_MUL_QUANT_GIVEN, oq=nvfp4_tensor(FAKE, FAKE, 0)) == m.ERR_NULL   # scale is read
    assert call(N=100) == m.ERR_SHAPE
    assert call(off=None) == m.ERR_NULL
    assert call(out=None) == m.ERR_NULL
    assert call(epi=m.EPI_SILU_MUL_REQUANT, w1=nvfp4_tensor(0, 0, 0)) == m.ERR_NULL
    assert call(rows=FAKE + 2) == m.ERR_ALIGN
    assert call(M=0) == m.OK
    s = _size()
    z = nvfp4_tensor(0, 0, 0)
    assert f(z, None, None, 64, 32768, z, z, 2048, 4096, m.EPI_SILU_MUL_REQUANT, None, m.F32, 2048, z, None,
             ctypes.byref(s), None) == m.OK
    assert s.value >= 32768 * 2048 * 4
    s2 = _size()
    assert f(z, None, None, 64, 32768, z, z, 2048, 4096, m.EPI_SILU_MUL_QUANT_GIVEN, None, m.F32, 2048, z, None,
             ctypes.byref(s2), None) == m.OK
    assert s2.value == 32768 * 4096 * 2                   # no float32 GLU output with a given scale


@no_gpu
def test_valid_calls_report_missing_device_and_launch_nothing():
    before = m.lib.nvfp4_launch_count()
    sz = ctypes.c_size_t(1 << 20)
    assert m.lib.nvfp4_quantize_act(FAKE, m.BF16, 4, 32, 32, _t(), 0, FAKE, ctypes.byref(sz), None) == m.ERR_DEVICE
    big = ctypes.c_size_t(1 << 24)
    assert m.lib.nvfp4_gemm(_t(), _t(), 4, 8, 128, FAKE, m.F32, 8, None, FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_mlp_gu_act(_t(), _t(), _t(), 4, 128, 128, _t(), FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_mlp_down(_t(), _t(), 4, 128, 64, FAKE, m.F32, 64, None, FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_mlp_gu_act_static(_t(), _t(), _t(), 4, 128, 128, _t(), FAKE, ctypes.byref(big),
                                         None) == m.ERR_DEVICE
    assert m.lib.nvfp4_mlp_down_quant(_t(), _t(), 4, 128, 64, _t(), FAKE, ctypes.byref(big), None) == m.ERR_DEVICE
    assert m.lib.nvfp4_launch_count() == before


def test_timing_window_validation():
    lib = m.lib
    n, d, ms = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_double()
    out = (ctypes.byref(n), ctypes.byref(d), ctypes.byref(ms))
    assert lib.nvfp4_timing_begin(-1, 8) == m.ERR_ARG
    assert lib.nvfp4_timing_begin(7, 8) == m.ERR_ARG                  # one past the last class
    assert lib.nvfp4_timing_begin(m.KC_GEMM_GLU, 0) == m.ERR_ARG
    assert lib.nvfp4_timing_begin(m.KC_GEMM_GLU, (1 << 20) + 1) == m.ERR_ARG
    assert lib.nvfp4_timing_end(*out) == m.ERR_ARG                      # no window open
    assert lib.nvfp4_timing_end(None, out[1], out[2]) == m.ERR_NULL
    st = lib.nvfp4_timing_begin(m.KC_GEMM_GLU, 4)
    if st == m.OK:                                                       # events available
        assert lib.nvfp4_timing_begin(m.KC_EXPAND, 4) == m.ERR_ARG      # one window at a time
        assert lib.nvfp4_timing_end(*out) == m.OK
        assert (n.value, d.value, ms.value) == (0, 0, 0.0)
    else:                                                                # no device: events cannot be made
        assert st == m.ERR_LAUNCH
        assert lib.nvfp4_timing_end(*out) == m.ERR_ARG


def test_moe_route_and_combine_validation():
    lib = m.lib
    sz = ctypes.c_size_t(1 << 20)
    r = lib.nvfp4_moe_route
    assert r(FAKE, 16, 0, 1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_ARG      # E < 1
    assert r(FAKE, 16, 8, 9, 8, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_ARG      # k > E
    assert r(FAKE, 16, 64, 17, 64, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_ARG   # k > 16
    assert r(FAKE, 16, 5000, 2, 5000, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_ARG
    assert r(FAKE, 16, 8, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_SHAPE    # ld < E
    assert r(FAKE, -1, 8, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sz), None) == m.ERR_SHAPE
    q = ctypes.c_size_t(0)
    assert r(None, 4096, 64, 8, 64, None, None, None, None, None, ctypes.byref(q), None) == m.OK
    assert q.value >= 2 * 4096 * 8 * 4 + 64 * 64 * 4                                                    # ids, ranks, counts
    small = ctypes.c_size_t(q.value - 1)
    assert r(FAKE, 4096, 64, 8, 64, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(small), None) == m.ERR_WORKSPACE
    z = ctypes.c_size_t(1 << 20)
    assert r(FAKE, 0, 64, 8, 64, None, None, None, None, FAKE, ctypes.byref(z), None) == m.OK           # T = 0
    big = lambda: ctypes.byref(ctypes.c_size_t(1 << 20))                                               # noqa: E731
    assert r(None, 16, 8, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big(), None) == m.ERR_NULL
    assert r(FAKE + 2, 16, 8, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big(), None) == m.ERR_ALIGN
    c = lib.nvfp4_moe_combine
    assert c(FAKE, 7, 64, FAKE, FAKE, 16, 2, 64, FAKE, m.F32, 64, None) == m.ERR_ARG                   # dtype
    assert c(FAKE, m.BF16, 64, FAKE, FAKE, 16, 0, 64, FAKE, m.F32, 64, None) == m.ERR_ARG              # k
    assert c(FAKE, m.BF16, 64, FAKE, FAKE, 16, 2, 60, FAKE, m.F32, 64, None) == m.ERR_SHAPE            # N % 8
    assert c(FAKE, m.BF16, 32, FAKE, FAKE, 16, 2, 64, FAKE, m.F32, 64, None) == m.ERR_SHAPE            # ld < N
    assert c(FAKE, m.BF16, 64, FAKE, FAKE, 0, 2, 64, FAKE, m.F32, 64, None) == m.OK                    # T = 0
    assert c(None, m.BF16, 64, FAKE, FAKE, 16, 2, 64, FAKE, m.F32, 64, None) == m.ERR_NULL
    assert c(FAKE, m.BF16, 68, FAKE, FAKE, 16, 2, 64, FAKE, m.F32, 64, None) == m.ERR_ALIGN            # row stride


def test_rmsnorm_quantize_validation():
    f = m.lib.nvfp4_rmsnorm_quantize_act
    big = lambda: ctypes.byref(ctypes.c_size_t(1 << 24))                                               # noqa: E731
    assert f(FAKE, 7, 4, 32, 32, FAKE, 1e-6, _t(), FAKE, big(), None) == m.ERR_ARG                     # dtype
    assert f(FAKE, m.BF16, 4, 32, 32, FAKE, -1.0, _t(), FAKE, big(), None) == m.ERR_ARG                # eps < 0
    assert f(FAKE, m.BF16, 4, 32, 32, FAKE, float("nan"), _t(), FAKE, big(), None) == m.ERR_ARG        # eps NaN
    assert f(FAKE, m.BF16, 4, 24, 24, FAKE, 1e-6, _t(), FAKE, big(), None) == m.ERR_SHAPE              # cols % 16
    assert f(FAKE, m.BF16, 4, 32, 16, FAKE, 1e-6, _t(), FAKE, big(), None) == m.ERR_SHAPE              # ld < cols
    q = ctypes.c_size_t(0)
    assert f(None, m.BF16, 1000, 5120, 5120, None, 1e-6, _t(0, 0, 0), None, ctypes.byref(q), None) == m.OK
    assert q.value >= 1000 * 4 + 4096 * 4
    assert f(FAKE, m.BF16, 0, 32, 32, None, 1e-6, _t(0, 0, 0), FAKE, big(), None) == m.OK              # rows = 0
    assert f(FAKE, m.BF16, 4, 32, 32, None, 1e-6, _t(), FAKE, big(), None) == m.ERR_NULL                # gamma
    assert f(FAKE, m.BF16, 4, 32, 32, FAKE + 4, 1e-6, _t(), FAKE, big(), None) == m.ERR_ALIGN          # gamma align
