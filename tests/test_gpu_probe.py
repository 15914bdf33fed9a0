"""The achievable-bandwidth probe (a measurement aid, not part of the method)
reads every word of its buffer exactly once."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_stream_read_sums_every_word_once():
    import routed_decode_attention_amd as rda
    n = (1 << 24) + 3  # three words past the last whole 16-byte granule
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    sink = torch.full((512,), float("nan"), dtype=torch.float32, device="cuda")
    rda.basiskv_stream_read(src, sink)
    torch.cuda.synchronize()
    assert float(sink.double().sum()) == n
    # distinct small integers: each word counted once, whatever its offset
    m = 4097 * 4 + 2
    vals = torch.arange(m, dtype=torch.int64) % 7
    src = vals.to(torch.float32).cuda()
    sink = torch.full((3,), float("nan"), dtype=torch.float32, device="cuda")
    rda.basiskv_stream_read(src, sink)
    torch.cuda.synchronize()
    assert float(sink.double().sum()) == int(vals.sum())
