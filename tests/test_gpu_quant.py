"""Device quantiser vs the oracle: codes, scales and global scale bit-exact."""
import numpy as np
import pytest
import torch

from oracle import quant
from synthetic import bf16_bits_to_f32, bf16_normal, outlier_channels
from tests.gpu_util import announce, assert_nvfp4_equal, dev_quantize, require_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


ACT_CASES = [
    # name, rows, cols, seed, outlier seed
    ("gemm_activation_16x256", 16, 256, 1001, None),
    ("decode_T1_5120", 1, 5120, 2001, None),
    ("decode_T5_5120", 5, 5120, 2001, None),
    ("ragged_37x512", 37, 512, 7, None),
    ("single_block_row", 3, 16, 8, None),
    ("prefill_1024x5120_outliers", 1024, 5120, 3001, 3005),
]


@pytest.mark.parametrize("name,rows,cols,seed,oseed", ACT_CASES, ids=[c[0] for c in ACT_CASES])
def test_quantize_bf16_activation_bit_exact(name, rows, cols, seed, oseed):
    announce(f"quantize bf16 {name}")
    outl = outlier_channels(oseed, cols) if oseed else None
    bits = bf16_normal(seed, (rows, cols), outliers=outl)
    got = to_host(dev_quantize(bits))
    ref = quant.quantize(bf16_bits_to_f32(bits))
    assert_nvfp4_equal(got, ref, name)


def _wide_range_f32(seed, rows, cols):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-6, 3, (rows, cols))).astype(np.float32)
    x[0, :16] = 0.0                       # all-zero block
    x[0, 16:32] = -0.0                    # negative zeros
    x[1, :16] *= 1e-7                     # tiny block: subnormal or zero E4M3 scale
    x[2, 32:48] = 1e-30                   # denormal-free tiny constant
    return x


def test_quantize_f32_wide_dynamic_range_bit_exact():
    announce("quantize f32 wide range 64x1024")
    x = _wide_range_f32(3, 64, 1024)
    got = to_host(dev_quantize(x))
    assert_nvfp4_equal(got, quant.quantize(x), "wide range")


def test_quantize_constructed_ties_bit_exact():
    announce("quantize constructed ties")
    # gs == 1 (2688 in the tensor); blocks with block-scale ties and element ties
    x = np.zeros((4, 128), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = 6 * 1.0625
    x[0, 32] = 6 * 1.1875
    x[0, 48:64] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.0]
    x[1, :16] = 6 * 4.5 * 2.0 ** -9         # r = 4.5 * 2^-9: subnormal tie, codes 4|5 -> 4
    x[2, :16] = np.float32(6 * 2.0 ** -10)  # r = 2^-10: tie between E4M3 0 and 2^-9
    x[3, :16] = np.float32(6 * 3 * 2.0 ** -11)  # r = 1.5 * 2^-9: tie between codes 1 and 2
    got = to_host(dev_quantize(x))
    ref = quant.quantize(x)
    assert ref.gs == np.float32(1.0)
    assert_nvfp4_equal(got, ref, "ties")


def test_quantize_given_global_scale():
    announce("quantize GS_GIVEN")
    bits = bf16_normal(77, (33, 256))
    x = bf16_bits_to_f32(bits)
    for gs in (np.float32(1e-3), np.float32(2.0 ** -12), np.float32(0.37)):
        got = to_host(dev_quantize(bits, gs_mode=1, gs=gs))
        assert_nvfp4_equal(got, quant.quantize(x, gs=gs), f"given gs {gs}")


def test_quantize_weights_sampled_rows_full_size():
    # a full 17408 x 5120 weight (N(0, 0.02)): global scale from the whole
    # matrix, rows checked on a sample (quantisation is row-local given gs)
    announce("quantize weight 17408x5120 (sampled rows)")
    bits = bf16_normal(3002, (17408, 5120), sigma=0.02)
    x = bf16_bits_to_f32(bits)
    q = dev_quantize(bits)
    gs = quant.global_scale(x)
    got = to_host(q)
    assert got.gs == gs
    rows = np.random.default_rng(0).choice(17408, 256, replace=False)
    rows = np.concatenate([[0, 17407], rows])
    ref = quant.quantize(x[rows], gs=gs)
    assert_nvfp4_equal(quant.NVFP4(got.codes[rows], got.scales[rows], got.gs, len(rows), 5120), ref, "weight rows")


def test_quantize_zero_rows_is_a_noop():
    import mlp_prefill_amd as m
    announce("quantize zero rows")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q = m.NVFP4.empty(1, 256)
    q.gscale.fill_(-7.0)
    m.nvfp4_quantize_act(x, q)
    torch.cuda.synchronize()
    assert q.gscale.item() == -7.0


def test_quantize_strided_rows():
    import mlp_prefill_amd as m
    announce("quantize row stride > cols")
    bits = bf16_normal(91, (9, 384))
    full = m.bf16_from_bits(bits)
    view = full[:, 64:320]                  # ld 384, cols 256, 128-byte aligned start
    q = m.NVFP4.empty(9, 256)
    m.nvfp4_quantize_act(view, q)
    ref = quant.quantize(bf16_bits_to_f32(bits)[:, 64:320])
    assert_nvfp4_equal(to_host(q), ref, "strided")
