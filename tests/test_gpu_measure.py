"""GPU check of the streaming read used to measure the device's practical HBM
read rate (bench.py --ceiling): its XOR of all 32-bit words equals numpy's on
the same seeded bytes, at the measured 128 MiB size, at a size that ends in a
partial grid-stride step, and for a single 16-byte chunk; an initial value in
the result word is XOR-ed, not overwritten."""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("nbytes", [16, 16 * 1_000_003, 128 << 20])
def test_stream_read_xor_matches_numpy(nbytes):
    _say("stream_read", nbytes)
    g = np.random.default_rng(nbytes % 1000)
    host = g.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    x = torch.from_numpy(host.view(np.int32)).cuda()
    got = mi.stream_read(x)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert np.uint32(got.cpu().numpy().view(np.uint32)[0]) == want
    seed = torch.tensor([0x5A5A5A5A], dtype=torch.int32, device="cuda")
    mi.stream_read(x, xor_out=seed)
    torch.cuda.synchronize()
    assert np.uint32(seed.cpu().numpy().view(np.uint32)[0]) == want ^ np.uint32(0x5A5A5A5A)
