"""The read-bandwidth probe reads every word it is given (MI355X only): its per-workgroup
XOR equals the XOR of the words a workgroup's threads cover, on a buffer with a ragged
tail."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_read_probe_reads_every_word():
    from bit_kv_cache_oscar_amd import _lib as L

    blocks = L.lib().oscar_read_probe_words()
    stride = blocks * 256  # 16-byte words per grid sweep
    n16 = 3 * stride + 12345
    words = np.random.default_rng(4).integers(0, 2 ** 32, (n16, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).reshape(-1).copy()).cuda()
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    print("[case] read probe", n16, "words", flush=True)
    L.oscar_read_probe(buf, out)
    got = out.cpu().numpy().view(np.uint32)
    # 16-byte word i is read by workgroup (i % stride) // 256
    owner = (np.arange(n16) % stride) // 256
    x = np.bitwise_xor.reduce(words, axis=1)
    want = np.zeros(blocks, np.uint32)
    np.bitwise_xor.at(want, owner, x)
    assert np.array_equal(got, want)
