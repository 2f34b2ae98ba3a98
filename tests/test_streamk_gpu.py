"""GPU parity of the persistent stream-K schedule ("Operator & Runtime"
§5.5.4, §5.2.4): every output element against the oracle, on shapes whose
tiles are split between workgroups in two or three pieces, whose tile count is
below, equal to or above the CU count, with edge tiles, batches, and fewer
units than CUs; repeated calls give the same bits."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import amax_bf16, check_bf16, check_f32, dev_bf16, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[streamk] {msg}", flush=True)


@pytest.fixture
def force_streamk(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)
    monkeypatch.setenv("GEMM_FORCE_STREAMK", "1")
    return monkeypatch


@pytest.mark.parametrize("cfg", ["bf16_256x256", "bf16_256x192"])
@pytest.mark.parametrize("M,N,K,batch,out", [
    (1024, 12288, 4096, 1, "bf16"),     # the FFN projection: 192 or 256 tiles, two pieces per split tile
    (512, 768, 4096, 1, "f32"),         # 6 or 8 tiles over 256 CUs: many pieces per tile
    (300, 712, 1024, 2, "bf16"),        # edge tiles (masked variant), a batch of 2
    (256, 256, 64, 1, "f32"),           # 2 units for 256 CUs: a grid of 2
    (2048, 2048, 2048, 1, "bf16"),      # 64 or 88 tiles
])
def test_streamk_matches_oracle(oracle_mod, force_streamk, cfg, M, N, K, batch, out):
    _say(f"{cfg} {batch}x{M}x{N}x{K} -> {out}")
    force_streamk.setenv("GEMM_FORCE_CONFIG", cfg)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, batch=batch, c_type=1 if out == "f32" else 0)
    assert st == 0 and plan.streamk == 1 and plan.name == cfg.encode(), (st, plan.name)
    g = np.random.default_rng([M, N, K, batch, 77])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    od = torch.bfloat16 if out == "bf16" else torch.float32
    dA, dB = dev_bf16(A), dev_bf16(B)
    C = g5.gemm_bf16_batched(dA, dB, out_dtype=od, workspace=ws())
    C2 = g5.gemm_bf16_batched(dA, dB, out_dtype=od, workspace=ws())
    assert torch.equal(C.view(torch.int16 if out == "bf16" else torch.int32),
                       C2.view(torch.int16 if out == "bf16" else torch.int32)), "not deterministic"
    ref = oracle_mod.gemm_bf16_batched(A, B)
    host = host_values(C)
    for b in range(batch):
        if out == "bf16":
            check_bf16(host[b], ref[b], K, f"batch {b}")
        else:
            check_f32(host[b], ref[b], K, amax_bf16(A[b]), amax_bf16(B[b]), f"batch {b}")
