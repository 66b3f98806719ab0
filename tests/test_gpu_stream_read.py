"""The measurement read (w4a16_stream_read), through the C ABI: every 16-byte
unit of each of its three ranges is read -- a single nonzero unit placed
anywhere in any range decides the store, and nothing else does."""
import pytest
import torch

import weight_only_int4_02_amd as w4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("sizes", [(16, 0, 0), (4096, 16, 48), (1 << 20, 4096, 1024),
                                   (48 << 20, 1 << 20, 512 << 10)])
def test_each_unit_of_each_range_is_read(sizes):
    bufs = [torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda") for n in sizes]
    views = [b[:n] for b, n in zip(bufs, sizes) if n]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k, v in enumerate(views):
        for unit in (0, v.numel() // 16 // 2, v.numel() // 16 - 1):
            v.view(torch.int32).zero_()
            words = v.view(torch.int32)[unit * 4:unit * 4 + 4]
            words.copy_(torch.tensor([1, 2, 4, 8 << k], dtype=torch.int32))
            key = 1 ^ 2 ^ 4 ^ (8 << k)
            sink.fill_(-1)
            w4.stream_read(views, sink, key=key + 1 if key + 1 != 0 else key + 2)
            torch.cuda.synchronize()
            assert int(sink.item()) == -1, "stored without a matching unit"
            w4.stream_read(views, sink, key=key)
            torch.cuda.synchronize()
            assert int(sink.item()) == key, f"range {k} unit {unit} not read"
