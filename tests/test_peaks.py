"""The achievable-peak measurements (include/ttt_peaks.h).

Without a GPU: the library exports what the header declares, and argument
errors return their status before any launch.  On the GPU: the copy is exact,
and the matrix-core issue loop returns the exact integer result its header
documents -- which also pins the v_mfma_f32_16x16x32_bf16 lane layout (A at
[l%16][8(l/16)+s], B at [8(l/16)+s][l%16], D at [4(l/16)+r][l%16]) that every
matrix-core kernel here relies on; the fp32 vector loop returns its exact
documented sums.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import test_sequence_layer_amd as ttt
from test_sequence_layer_amd import peaks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPE, NULL, ALIGN, ALIAS, OK = 2, 1, 6, 5, 0
GB = 1 << 30


def test_header_declares_what_the_library_exports():
    src = open(os.path.join(ROOT, "include", "ttt_peaks.h")).read()
    declared = sorted(set(re.findall(r"^\s*[a-z_0-9]+\s*\*?\s*(ttt_[a-z_0-9]+)\s*\(", src, re.M)))
    assert declared == sorted(peaks.PEAK_EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ttt.LIB_PATH], capture_output=True, text=True).stdout
    for sym in declared:
        assert re.search(rf"\bT {sym}$", out, re.M), sym


def test_argument_errors_before_launch():
    L = peaks._plib()
    assert L.ttt_peak_copy(GB, 2 * GB, 24, None) == SHAPE        # not a multiple of 16
    assert L.ttt_peak_copy(GB, 2 * GB, -16, None) == SHAPE
    assert L.ttt_peak_copy(GB, 2 * GB, 0, None) == OK            # nothing to do
    assert L.ttt_peak_copy(None, 2 * GB, 64, None) == NULL
    assert L.ttt_peak_copy(GB + 8, 2 * GB, 64, None) == ALIGN
    assert L.ttt_peak_copy(GB, GB + 32, 64, None) == ALIAS
    assert L.ttt_peak_mfma_bf16(GB, 0, 10, None) == SHAPE
    assert L.ttt_peak_mfma_bf16(GB, 4, -1, None) == SHAPE
    assert L.ttt_peak_mfma_bf16(None, 4, 10, None) == NULL
    assert L.ttt_peak_mfma_bf16(GB + 4, 4, 10, None) == ALIGN
    assert peaks.mfma_bf16_flops(512, 20000) == 512 * 4 * 20000 * 8 * 2 * 16 * 16 * 32
    assert peaks.mfma_bf16_flops(0, 1) == -1
    assert L.ttt_peak_valu_f32(GB, 0, 10, None) == SHAPE
    assert L.ttt_peak_valu_f32(GB, 4, -1, None) == SHAPE
    assert L.ttt_peak_valu_f32(GB, 4, 300001, None) == SHAPE     # past the exactness bound
    assert L.ttt_peak_valu_f32(None, 4, 10, None) == NULL
    assert L.ttt_peak_valu_f32(GB + 2, 4, 10, None) == ALIGN
    assert peaks.valu_f32_flops(2048, 50000) == 2048 * 256 * 50000 * 16 * 2
    assert peaks.valu_f32_flops(1, -1) == -1


def _expected_mfma(blocks, iters):
    """out[4 (256 q + t) + r] = 8 iters (A B)[4 ((t % 64) // 16) + r][t % 16], from the operand
    values the header gives per lane and slot, placed by the documented lane layout."""
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for lane in range(64):
        for s in range(8):
            A[lane % 16, 8 * (lane // 16) + s] = (lane + s) % 5 - 2
            B[8 * (lane // 16) + s, lane % 16] = (3 * lane + s) % 7 - 3
    C = A @ B
    t = np.arange(256)
    lane = t % 64
    per_thread = np.stack([8 * iters * C[4 * (lane // 16) + r, lane % 16] for r in range(4)], axis=1)
    return np.tile(per_thread.reshape(-1), blocks)


@pytest.mark.gpu
def test_copy_is_exact():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(3)
    for n in (16, 4096 + 16, 3 * (1 << 20) + 48):  # ragged against the 256-thread blocks
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0", generator=g)
        dst = torch.zeros_like(src)
        peaks.copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), n


@pytest.mark.gpu
@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 37), (2, 10000)])
def test_mfma_loop_is_exact(blocks, iters):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    out = torch.full((blocks * 1024,), float("nan"), dtype=torch.float32, device="cuda:0")
    peaks.mfma_bf16(out, blocks, iters)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), _expected_mfma(blocks, iters))


@pytest.mark.gpu
def test_measurements_are_plausible():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw = peaks.measure_hbm_copy(nbytes=256 << 20, warmup=3, reps=5)
    tf = peaks.measure_mfma_bf16(blocks=512, iters=2000, warmup=1, reps=2)
    vf = peaks.measure_valu_f32(blocks=1024, iters=5000, warmup=1, reps=2)
    print(f"copy {bw:.0f} GB/s, bf16 MFMA {tf:.0f} TFLOP/s, fp32 v_fma {vf:.1f} TFLOP/s", flush=True)
    assert 1000 < bw < 8000 * 1.05
    assert 300 < tf < 2517 * 1.05
    assert 10 < vf < 157.3 * 1.05


@pytest.mark.gpu
def test_valu_loop_is_exact():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for blocks, iters in ((3, 0), (5, 1000), (2, 300000)):
        out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda:0")
        peaks.valu_f32(out, blocks, iters)
        torch.cuda.synchronize()
        t = np.arange(blocks * 256) % 256
        assert np.array_equal(out.cpu().numpy(), (120 + 16 * iters * (t % 4)).astype(np.float32)), (blocks, iters)
