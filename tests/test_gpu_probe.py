"""The two streaming-read measurement aids run over sizes that are not whole
multiples of their workgroup shares and write nothing for this input."""
import pytest
import torch

import compressed_domain_decode_amd as tq


@pytest.mark.gpu
@pytest.mark.parametrize("resident", [False, True])
@pytest.mark.parametrize("nbytes", [16, 48 * 1024 + 16, 3 * 1024 * 1024 + 4096 + 48])
def test_stream_read_runs_and_writes_nothing(resident, nbytes):
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    print(f"stream read: resident={resident} bytes={nbytes}", flush=True)
    tq.tq_stream_read(buf, sink, resident=resident)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
