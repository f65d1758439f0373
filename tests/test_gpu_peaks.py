"""The measurement library (libglm_peaks.so) on the GPU: each probe stays
within what the hardware can do at the clock the probe itself observed, the
layered step probe is ordered as its modes imply, and bad arguments are
rejected with hipErrorInvalidValue (1) before anything runs.

Bounds:
  * MFMA loop: the published 2.5166 PFLOP/s bf16 and 5.033 PFLOP/s fp8 dense
    rates hold at 2400 MHz, so flops per shader-clock cycle cannot exceed
    peak / 2400 MHz.  One wave samples the clock of its own XCD while the
    others may run a little slower, hence the 10% allowance.
  * GEMM step, MFMAs only: each of a SIMD's two waves issues 32
    v_mfma_f32_32x32x16_bf16 (32 cycles each) per step, so no step takes
    fewer than 2048 cycles.  Adding copies or fragment reads to the same step
    cannot make it cheaper.
  * HBM read: not above the published 8 TB/s.
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PEAK_BF16 = 2.5166e15
PEAK_FP8 = 5.0332e15
PEAK_CLOCK_HZ = 2.4e9
INVALID = 1  # hipErrorInvalidValue

vp, i32, f64p, f32p = (ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                       ctypes.POINTER(ctypes.c_float))


@pytest.fixture(scope="module")
def peaks():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    path = os.path.join(ROOT, "sparse_moe_transformer_glm_amd", "libglm_peaks.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "python -m sparse_moe_transformer_glm_amd.build")
    torch.cuda.set_device(0)
    L = ctypes.CDLL(path)
    L.glm_peak_mfma.argtypes = [i32, i32, i32, vp, f32p, f64p, f64p, vp]
    L.glm_peak_hbm_read.argtypes = [vp, ctypes.c_size_t, i32, vp, f32p, vp]
    L.glm_peak_gemm_step.argtypes = [i32, i32, vp, vp, f64p, f64p, vp]
    L.glm_peak_clock_probe.argtypes = [ctypes.c_double, i32, i32, vp, vp]
    stream = torch.cuda.current_stream().cuda_stream
    scratch = torch.empty(16 + 4096 * 512 * 4, dtype=torch.uint8, device="cuda")
    return L, stream, scratch


@pytest.mark.parametrize("fp8, peak", [(0, PEAK_BF16), (1, PEAK_FP8)], ids=["bf16", "fp8"])
def test_mfma_loop_within_rate_at_its_clock(peaks, fp8, peak):
    L, stream, scratch = peaks
    ms, flops, mhz = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
    st = L.glm_peak_mfma(fp8, 20000, 2, scratch.data_ptr(), ctypes.byref(ms),
                         ctypes.byref(flops), ctypes.byref(mhz), stream)
    assert st == 0
    assert 500.0 < mhz.value < 3000.0, mhz.value
    per_cycle = flops.value / (ms.value * 1e-3) / (mhz.value * 1e6)
    bound = peak / PEAK_CLOCK_HZ
    print(f"fp8={fp8}: {flops.value / (ms.value * 1e-3) / 1e12:.1f} TFLOP/s at "
          f"{mhz.value:.0f} MHz, {per_cycle / bound:.3f} of the per-cycle peak")
    assert per_cycle <= 1.10 * bound
    assert per_cycle >= 0.70 * bound  # a loop of independent MFMAs runs near the rate


def _step(L, stream, scratch, src, mode, iters=2000):
    us, mhz = ctypes.c_double(), ctypes.c_double()
    st = L.glm_peak_gemm_step(mode, iters, src.data_ptr(), scratch.data_ptr(), ctypes.byref(us),
                              ctypes.byref(mhz), stream)
    assert st == 0, (mode, st)
    assert us.value > 0 and 500.0 < mhz.value < 3000.0
    return us.value * mhz.value  # shader-clock cycles per step


def test_gemm_step_modes_ordered(peaks):
    L, stream, scratch = peaks
    src = torch.ones(512 * 12288 // 2, dtype=torch.bfloat16, device="cuda")
    cyc = {m: _step(L, stream, scratch, src, m) for m in range(7)}
    print({m: round(c) for m, c in cyc.items()})
    mfma = cyc[0]
    assert 0.97 * 2048 <= mfma <= 1.25 * 2048
    for m in (2, 3, 4, 5, 6):  # MFMAs plus copies and / or reads
        assert cyc[m] >= 0.97 * mfma, (m, cyc[m], mfma)
    assert cyc[2] >= 0.97 * cyc[1] and cyc[3] >= 0.97 * cyc[1]  # full steps include the copies


def test_hbm_read_below_published_peak(peaks):
    L, stream, scratch = peaks
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ms = ctypes.c_float()
    assert L.glm_peak_hbm_read(buf.data_ptr(), nbytes, 2, scratch.data_ptr(), ctypes.byref(ms),
                               stream) == 0
    gbs = nbytes / (ms.value * 1e-3) / 1e9
    print(f"{gbs:.0f} GB/s")
    assert 1000.0 < gbs <= 8000.0


def test_clock_probe_samples(peaks):
    L, stream, _ = peaks
    n = 64
    buf = torch.zeros(2 * n + 1, dtype=torch.int64, device="cuda")
    assert L.glm_peak_clock_probe(0.01, 100, n, buf.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    b = buf.cpu().tolist()
    count = b[2 * n]
    assert 2 <= count <= n
    mhz = 100.0 * (b[2 * (count - 1)] - b[0]) / (b[2 * (count - 1) + 1] - b[1])
    assert 500.0 < mhz < 3000.0, mhz


def test_bad_arguments_rejected(peaks):
    L, stream, scratch = peaks
    us, mhz, ms, fl = ctypes.c_double(), ctypes.c_double(), ctypes.c_float(), ctypes.c_double()
    src = torch.ones(512 * 12288 // 2, dtype=torch.bfloat16, device="cuda")
    s, p = src.data_ptr(), scratch.data_ptr()
    assert L.glm_peak_gemm_step(7, 2, s, p, ctypes.byref(us), ctypes.byref(mhz), stream) == INVALID
    assert L.glm_peak_gemm_step(-1, 2, s, p, ctypes.byref(us), ctypes.byref(mhz), stream) == INVALID
    assert L.glm_peak_gemm_step(0, 3, s, p, ctypes.byref(us), ctypes.byref(mhz), stream) == INVALID
    assert L.glm_peak_gemm_step(0, 2, None, p, ctypes.byref(us), ctypes.byref(mhz), stream) == INVALID
    assert L.glm_peak_mfma(0, 0, 2, p, ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(mhz),
                           stream) == INVALID
    assert L.glm_peak_mfma(0, 10, 0, p, ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(mhz),
                           stream) == INVALID
    assert L.glm_peak_hbm_read(s, 15, 1, p, ctypes.byref(ms), stream) == INVALID
    assert L.glm_peak_hbm_read(s, 1 << 20, 0, p, ctypes.byref(ms), stream) == INVALID
    assert L.glm_peak_clock_probe(0.0, 100, 8, p, stream) == INVALID
    assert L.glm_peak_clock_probe(11.0, 100, 8, p, stream) == INVALID
