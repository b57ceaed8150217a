"""The MFMA calibration kernel (moe_mfma_peak): its flop count, and its result
against the same products computed on the host.  Each wave's lane 0 sums column
0, rows 8g + q (g, q < 4), of its four accumulator chains of iters 32 x 32 x 16
products: with fixed operands (bf16 values of the lane id) the chains are
identical; with varied ones each chain alternates two of eight hashed pairs."""
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


def cal_bits(lane, j, i, ab):
    """The varied mode's operand bits (bf16): sign, exponent 2^-4 and mantissa from
    a 32-bit integer hash of (lane, pair j, element i, a or b)."""
    m = 0xFFFFFFFF
    h = ((lane * 0x9E3779B1) & m) ^ (((j * 8 + i) * 0x85EBCA77) & m) ^ ((ab * 0xC2B2AE3D) & m)
    h ^= h >> 15
    h = (h * 0x2C1B3C6D) & m
    h ^= h >> 12
    return 0x3D80 | (h & 0x807F)


def varied_operands(j):
    A = np.zeros((32, 16), np.uint16)
    B = np.zeros((16, 32), np.uint16)
    for lane in range(64):
        for i in range(8):
            k = 8 * (lane // 32) + i
            A[lane % 32, k] = cal_bits(lane, j, i, 0)
            B[k, lane % 32] = cal_bits(lane, j, i, 1)
    return bf16_bits_to_f32(A).astype(np.float64), bf16_bits_to_f32(B).astype(np.float64)


def test_mfma_peak_varied_result():
    """Varied operands: chain c takes pair c on even iterations and pair 4 + c on odd
    ones (an odd count, so the single-step tail runs too)."""
    iters = 63
    sink = torch.full((moe.MFMA_PEAK_SINK,), float("nan"), device="cuda")
    flops = moe.mfma_peak(iters, sink, varied=True)
    torch.cuda.synchronize()
    assert flops == 2048 * 4 * iters * 4 * 2 * 32 * 32 * 16
    ops = [varied_operands(j) for j in range(8)]
    n_even, n_odd = (iters + 1) // 2, iters // 2
    rows = [8 * g + q for g in range(4) for q in range(4)]
    want = 0.0
    scale = 0.0
    for c in range(4):
        (A0, B0), (A1, B1) = ops[c], ops[4 + c]
        C = n_even * (A0 @ B0) + n_odd * (A1 @ B1)
        want += C[rows, 0].sum()
        scale += n_even * (np.abs(A0) @ np.abs(B0))[rows, 0].sum() + n_odd * (np.abs(A1) @ np.abs(B1))[rows, 0].sum()
    got = bits(sink)
    assert np.all(np.abs(got - want) <= 1e-5 * scale), (got[:4], want, scale)


@pytest.mark.parametrize("nblocks", [3, 4096 * 2 + 5])
def test_hbm_read_peak_result(nblocks):
    """Entry w of the sink is the XOR of every 32-bit word of the 32 KiB blocks w, w + 4096, ... of the
    buffer (0 where there are none): the launch read every byte once, in the documented assignment."""
    words = np.random.default_rng(1234 + nblocks).integers(0, 2 ** 32, size=nblocks * 8192, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.full((moe.HBM_READ_SINK,), -1, dtype=torch.int32, device="cuda")
    got_bytes = moe.hbm_read_peak(buf, sink)
    torch.cuda.synchronize()
    assert got_bytes == nblocks * moe.HBM_READ_BLOCK
    per_block = np.bitwise_xor.reduce(words.reshape(nblocks, 8192), axis=1)
    want = np.zeros(moe.HBM_READ_SINK, np.uint32)
    for b in range(nblocks):
        want[b % moe.HBM_READ_SINK] ^= per_block[b]
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
