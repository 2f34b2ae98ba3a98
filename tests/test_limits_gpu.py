"""GPU parity at the library's size limits, through the C ABI: an operand
past 2 GiB (beyond the 32-bit buffer offsets of the ring kernels, so the
general kernel runs with 64-bit addressing) and a batch count past the
small-M path's grid limit (65535 entries)."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import check_bf16, check_f32, amax_bf16, dev_bf16, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)


def test_operand_over_2gib(oracle_mod):
    """A [270000, 4096] bf16 (2.2e9 bytes) times B [4096, 128]: A's rows are
    a seeded block of 4099 rows repeated (row i is block row i mod 4099, a
    period that no power-of-two addressing error preserves); rows on both
    sides of the 2^31-byte mark and the last row are compared with the
    oracle."""
    M, N, K, P = 270000, 128, 4096, 4099
    print(f"[limits] A {M}x{K} bf16, {M * K * 2 / 1e9:.2f} GB", flush=True)
    g = np.random.default_rng([gi.SEED_BASE + 8000])
    block = gi.to_bf16_bits(gi.normal(g, (P, K)))
    B = gi.to_bf16_bits(gi.normal(g, (K, N), 0.125))
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, a_addr=1 << 40, b_addr=2 << 40, c_addr=3 << 40)
    assert st == 0 and plan.variant == 0
    dA = dev_bf16(block).repeat(M // P + 1, 1)[:M]
    assert dA.is_contiguous() and dA.shape == (M, K)
    C = g5.gemm_bf16(dA, dev_bf16(B), workspace=ws())
    rows = np.array([0, 1, P - 1, P, 131071, 262143, 262144, 262145, 265000, M - 1])
    got = host_values(C[torch.from_numpy(rows).cuda()])
    ref = oracle_mod.gemm_bf16(np.ascontiguousarray(block[rows % P]), B)
    check_bf16(got, ref, K, "rows across the 2 GiB mark")
    del dA, C
    torch.cuda.empty_cache()


def test_batch_past_small_m_grid(oracle_mod):
    """70000 entries of [1, 32] . [32, 16] (small M, but more entries than
    the small-M grid's y dimension holds): the tiled kernels run it; entries
    at both ends and around 65535 are compared with the oracle."""
    batch, M, N, K = 70000, 1, 16, 32
    g = np.random.default_rng([gi.SEED_BASE + 8100])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    C = g5.gemm_bf16_batched(dev_bf16(A), dev_bf16(B), out_dtype=torch.float32, workspace=ws())
    host = host_values(C)
    for b in (0, 1, 65534, 65535, 65536, batch - 1):
        ref = oracle_mod.gemm_bf16(A[b], B[b])
        check_f32(host[b], ref, K, amax_bf16(A[b]), amax_bf16(B[b]), f"entry {b}")
