"""The streaming-read reference (include/pkv_ref.h) reads every byte: the
XOR of its per-wavefront words is the XOR of the buffer's 32-bit words."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 * 16 + 48, 7), (1 << 22, 64),
                                           ((1 << 22) + 16 * 1000, 4096)])
def test_stream_read_touches_every_word(nbytes, blocks):
    g = torch.Generator().manual_seed(nbytes + blocks)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    src = host.cuda()
    sink = pkv.pkv_ref_stream_read(src, blocks)
    torch.cuda.synchronize()
    words = int(pkv.lib().pkv_ref_stream_sink_words(blocks))
    got = np.bitwise_xor.reduce(sink[:words].cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
