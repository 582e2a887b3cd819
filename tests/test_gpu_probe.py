"""The streaming-read probe (include/bnbx_probe.h) reads every byte of both
buffers exactly once: the XOR of the words it reports equals the XOR of all
words of the two buffers, computed on the host.  The sizes include a single
16-byte unit, unit counts that do not fill a workgroup's last round, and the
decode GEMV's weight-side byte counts (packed weights, then block codes) for
4096x4096 and 11008x4096."""

import numpy as np
import pytest
import torch

import dequant_gemm_nf4_amd as bnbx

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("a_bytes,b_bytes", [
    (16, 0), (48, 32), (16 * 2049, 16 * 7),
    (4096 * 4096 // 2, 4096 * 4096 // 64),
    (11008 * 4096 // 2, 11008 * 4096 // 64),
])
def test_probe_reads_every_word_once(a_bytes, b_bytes):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(a_bytes + 3 * b_bytes)
    a = torch.randint(-2**31, 2**31 - 1, (a_bytes // 4,), generator=g, dtype=torch.int32, device=dev)
    b = (torch.randint(-2**31, 2**31 - 1, (b_bytes // 4,), generator=g, dtype=torch.int32, device=dev)
         if b_bytes else None)
    sink = torch.zeros(bnbx.BNBX_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    print(f"probe a={a_bytes} b={b_bytes}", flush=True)
    bnbx.bnbx_probe_stream_read(a, a_bytes, b, b_bytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(a.cpu().numpy().view(np.uint32))
    if b is not None:
        want ^= np.bitwise_xor.reduce(b.cpu().numpy().view(np.uint32))
    assert got == want
