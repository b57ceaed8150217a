"""The MFMA calibration kernel (moe_mfma_peak): its flop count, and its result
against the same product computed on the host (each wave's lane 0 sums column
0, rows 8g + q (g, q < 4), of four identical accumulator chains of iters
32 x 32 x 16 products; the operands are fixed bf16 values of the lane id)."""
import numpy as np
import pytest
import torch

import top_routing_expert_gemm_amd as moe
from moe_gpu import bits, require_gpu
from synth import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def operands():
    """A [32, 16] and B [16, 32] as the kernel's lanes supply them: lane l gives
    A[l % 32, 8 (l // 32) + i] and B[8 (l // 32) + i, l % 32], i < 8."""
    A = np.zeros((32, 16), np.float32)
    B = np.zeros((16, 32), np.float32)
    for lane in range(64):
        for i in range(8):
            k = 8 * (lane // 32) + i
            A[lane % 32, k] = np.float32(1e-3) * np.float32((lane + i) & 7)
            B[k, lane % 32] = np.float32(1e-3) * np.float32((lane * 3 + i) & 7)
    rb = lambda m: bf16_bits_to_f32(f32_to_bf16_bits(m)).astype(np.float64)
    return rb(A), rb(B)


def test_mfma_peak_result_and_flops():
    iters = 64
    sink = torch.full((moe.MFMA_PEAK_SINK,), float("nan"), device="cuda")
    flops = moe.mfma_peak(iters, sink)
    torch.cuda.synchronize()
    assert flops == 2048 * 4 * iters * 4 * 2 * 32 * 32 * 16
    A, B = operands()
    C = iters * (A @ B)
    rows = [8 * g + q for g in range(4) for q in range(4)]
    want = 4 * C[rows, 0].sum()
    got = bits(sink)
    assert np.all(np.abs(got - want) <= 1e-5 * abs(want) + 1e-9), (got[:4], want)
