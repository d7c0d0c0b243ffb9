"""fa_read_probe (the streaming-read helper the bench times beside the paged
decode) reads every 32-bit word of its buffer exactly once: the sink ends as
its prior value XOR the XOR of all words, for sizes that fill the slabs of its
workgroups unevenly."""
import numpy as np
import pytest
import torch

import exact_attention_106_amd as fa


@pytest.mark.gpu
@pytest.mark.parametrize("n_bytes", [16, 4096 + 16, (1 << 20) + 48, 64 << 20])
def test_read_probe_reads_every_word_once(n_bytes):
    dev = torch.device("cuda", 0)
    rng = np.random.Generator(np.random.PCG64(n_bytes))
    words = rng.integers(0, 2**32, size=n_bytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    init = np.uint32(0x12345678)
    sink = torch.tensor([int(init.view(np.int32))], dtype=torch.int32, device=dev)
    fa.fa_read_probe(src, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(words, initial=np.uint32(0)) ^ init
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == expect
