"""The codebook-stream probe (measurement support for bench.py) runs and times itself."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import _lib, api  # noqa: E402


def test_stream_probe_runs():
    blocks, steps = 16, 2
    ws = api.Workspace(_lib.tcq_l16_stream_probe_bytes(blocks), "cuda")
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)  # torch creates the HIP events at their first record
    b.record(stream)
    _lib.tcq_l16_stream_probe(blocks, steps, ws.ptr, ws.nbytes, stream.cuda_stream,
                              a.cuda_event, b.cuda_event)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) > 0.0
