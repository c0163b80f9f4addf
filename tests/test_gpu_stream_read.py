"""The streaming-read instrument (df_stream_read) reads every byte it is
given: the XOR of its per-wave words equals the XOR of all 32-bit words of
the source, computed on the host, for sizes from empty to ragged multi-share
buffers."""
import numpy as np
import pytest
import torch

from dual_flow_transformer_amd import _abi
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 1008, 1 << 20, (64 << 20) + 4096 + 48, 300_000_016])
def test_stream_read_xor(nbytes):
    say(f"df_stream_read over {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes % 1000003)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (max(nbytes // 4, 1),), generator=g, dtype=torch.int32)[:nbytes // 4]
    src = words.cuda() if nbytes else torch.empty(4, dtype=torch.int32, device="cuda")
    out = torch.zeros(_abi.DF_STREAM_READ_OUT_WORDS, dtype=torch.int32, device="cuda")
    _abi.check(_abi.df_stream_read(src.data_ptr(), nbytes, out.data_ptr(), torch.cuda.current_stream().cuda_stream),
               "df_stream_read")
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32)) if nbytes else np.uint32(0)
    assert got == want


def test_stream_read_leaves_words_past_the_waves():
    """Wave w writes word w only: words from 4 x compute units on keep their contents."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    out = torch.full((_abi.DF_STREAM_READ_OUT_WORDS,), 7, dtype=torch.int32, device="cuda")
    _abi.check(_abi.df_stream_read(src.data_ptr(), src.numel() * 4, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream), "df_stream_read")
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[4 * cus:] == 7)
    assert np.bitwise_xor.reduce(o[:4 * cus].view(np.uint32)) == np.bitwise_xor.reduce(
        np.arange(1 << 16, dtype=np.uint32))
