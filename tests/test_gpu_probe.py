"""GPU check of the streaming-read probe (mxm_stream_xor, a measurement aid
of bench.py): it must read every byte it is given, so its XOR of all 32-bit
words equals numpy's, for both cache policies and ragged sizes."""

import numpy as np
import pytest
import torch

from _gpu import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 16384 * 3 + 16, 1 << 22, (1 << 26) + 1024])
@pytest.mark.parametrize("nt", [0, 1])
def test_stream_xor_reads_every_word(nbytes, nt):
    import mxfp4_moe_expert_route_amd as mm
    say("stream_xor", nbytes, "bytes, nontemporal" if nt else "bytes, default policy")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    seed = 0x5A5A1234
    res = torch.tensor([np.int32(np.uint32(seed).view(np.int32))], dtype=torch.int32, device=DEV)
    mm.mxm_stream_xor(src, res, nt)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host)) ^ seed
    assert (int(res.item()) & 0xFFFFFFFF) == want
