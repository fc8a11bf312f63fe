"""GPU test of the packed lm-head weight layout (ril_pack_lm_head): every element lands
where include/ril.h says, and the padding columns of the last vocabulary tile are zero.
The expected layout is built with plain tensor reshapes on the host."""

import numpy as np
import pytest
import torch

import invariant_rl_logprob_amd as ril

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,K", [(1000, 64), (2048, 256), (256, 32)])
def test_pack_layout(V, K):
    g = torch.Generator().manual_seed(V * 7 + K)
    w = torch.randint(-30000, 30000, (V, K), generator=g, dtype=torch.int32).to(torch.int16)
    packed = torch.full((ril.ril_lm_head_packed_bytes(V, K),), 0x55, dtype=torch.uint8, device="cuda")
    ril.ril_pack_lm_head(w.view(torch.bfloat16).cuda(), packed)
    torch.cuda.synchronize()
    got = packed.cpu().view(torch.int16).numpy()
    n_vt = (V + 255) // 256
    full = np.zeros((n_vt * 256, K), dtype=np.int16)
    full[:V] = w.numpy()
    # (c, k) -> block c/16, step k/32, lane ((k%32)/8)*16 + c%16, element k%8
    exp = full.reshape(n_vt * 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp)
