"""GPU check of the measurement helper attn_probe_stream: every work-group
streams its own slice and reports the first float of the slice's last 1 KB."""
import pytest
import torch

import blockwise_softmax_attention_amd as ba

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks", [1, 8, 512])
def test_stream_probe_reads_each_slice(blocks):
    n = 1 << 20                                   # 4 MiB of float32, exact integers
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    out = ba.attn_probe_stream(src, blocks)
    torch.cuda.synchronize()
    per_wg = n * 4 // blocks
    idx = torch.tensor([((b + 1) * per_wg - 1024) // 4 for b in range(blocks)], dtype=torch.float32)
    assert torch.equal(out.cpu(), idx)
