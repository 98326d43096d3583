"""The streaming-read diagnostic runs over whole and ragged buffer sizes
(smaller than the grid, not a multiple of the per-workgroup chunk) and
writes nothing when the data do not XOR to its fixed value."""

import pytest
import torch

import exact_tiled_attention_11_amd as fa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 4 * 1000, 4 * 2048 * 256 * 4 + 4 * 37, 1 << 26])
def test_stream_read_runs_and_leaves_sink(n_words):
    print(f"stream_read n_words={n_words}", flush=True)
    buf = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    fa.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7
