"""The streaming-read probe (a measurement utility beside the attention path)
runs through the C ABI, reads its whole buffer without writing its output
word, and reports a plausible rate."""
import pytest
import torch

import decode_attention_token_amd as kvq

pytestmark = pytest.mark.gpu


def test_stream_read_probe_runs_and_reads_at_a_plausible_rate():
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")     # 1 GiB, four times the MALL
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        kvq.kvq_stream_read_probe(buf, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        kvq.kvq_stream_read_probe(buf, out)
    e1.record()
    torch.cuda.synchronize()
    gbs = buf.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(f"  probe {gbs:.0f} GB/s over 1 GiB", flush=True)
    assert int(out.item()) == 0          # a buffer of ones never hits the store
    assert 500 < gbs < 8000              # below the 8 TB/s specification, far above a host copy
