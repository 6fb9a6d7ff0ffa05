"""The measurement utilities the benchmark compares the kernels with: the streaming read must
touch every byte it is asked to read (else its rate would overstate the ceiling), the copy must
copy them, and the flush must overwrite them."""
import numpy as np
import pytest
import torch

import paged_kv_cache_245_amd as pa
from gpu_support import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 12345])
def test_bench_read_touches_every_byte(nbytes):
    """pa_bench_read leaves, per workgroup, the XOR of the 32-bit words it read (low 23 bits);
    the XOR over the sink must equal the XOR of the whole buffer. Sizes: one 16-byte piece, a
    tail shorter than one unrolled iteration, and 64 MiB plus an odd tail."""
    say(f"  bench read {nbytes} bytes")
    rng = np.random.default_rng(nbytes % 1000 + 7)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    pa.pa_bench_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words) & np.uint32(0x007FFFFF)
    assert int(got) == int(want)


def test_bench_copy_and_flush():
    """pa_bench_copy copies every byte; pa_bench_flush overwrites every byte."""
    n = (8 << 20) + 16 * 77
    rng = np.random.default_rng(11)
    src = torch.from_numpy(rng.integers(-(1 << 31), 1 << 31, size=n // 4, dtype=np.int64).astype(np.int32)).cuda()
    dst = torch.zeros_like(src)
    pa.pa_bench_copy(dst, src, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    pa.pa_bench_flush(dst, n)
    torch.cuda.synchronize()
    assert not torch.equal(dst, src)
    # the overwrite pattern is a function of the 16-byte index only
    again = src.clone()
    pa.pa_bench_flush(again, n)
    torch.cuda.synchronize()
    assert torch.equal(again, dst)
