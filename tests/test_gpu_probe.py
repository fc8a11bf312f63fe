"""GPU test of the HBM read probe (benchmarking only): it reads every 16-byte chunk of the
buffer exactly once, so the XOR of its output words equals the XOR of all 32-bit words."""

import numpy as np
import pytest
import torch

import invariant_rl_logprob_amd as ril

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bytes", [16, 4096 + 48, (1 << 22) + 16 * 7])
def test_read_probe_touches_every_word_once(n_bytes):
    g = torch.Generator().manual_seed(n_bytes)
    host = torch.randint(0, 256, (n_bytes,), generator=g, dtype=torch.int32).to(torch.uint8)
    out = torch.zeros(ril.ril_hbm_read_probe_words(), dtype=torch.int32, device="cuda")
    ril.ril_hbm_read_probe(host.cuda(), out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy()[: n_bytes // 16 * 16].view(np.uint32))
    assert got == want
