"""The read-lane kernel runs, reads its buffer and writes nothing for ordinary
data (its sink is only written for one improbable folded value)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_lane_read_runs_and_leaves_sink():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd import dsa
    for n in (16, 4096 + 16, 3 << 20):
        buf = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        dsa.dsa_lane_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0
    with pytest.raises(dsa.DsaError):
        dsa.dsa_lane_read(torch.zeros(17, dtype=torch.uint8, device="cuda"), sink)
