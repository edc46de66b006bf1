"""The read-bandwidth probe reads every byte it is given: its per-row XOR of
32-bit words equals the host's, bit for bit, for one and two arrays, one and
four waves per row, rows shorter than one tile, rows with a ragged last tile
and the headline row size."""
import numpy as np
import pytest
import torch

import quantization_quality_eval_amd as qqe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _xor_rows(*arrays):
    out = np.zeros(arrays[0].shape[0], np.uint32)
    for a in arrays:
        out ^= np.bitwise_xor.reduce(a.view(np.uint32), axis=1)
    return out


@pytest.mark.parametrize("n_rows,row_words", [(1, 4), (5, 12), (37, 256), (9, 4 * 64 * 16 + 4 * 48),
                                              (16, 151936 // 2), (3, 262144 // 2 + 4)])
@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("waves", [1, 4])
def test_read_probe_checksums(n_rows, row_words, two, waves):
    g = np.random.default_rng(n_rows * 7 + row_words)
    ha = g.integers(0, 2 ** 32, (n_rows, row_words), dtype=np.uint32)
    hb = g.integers(0, 2 ** 32, (n_rows, row_words), dtype=np.uint32)
    a = torch.as_tensor(ha.view(np.int32), device=DEV)
    b = torch.as_tensor(hb.view(np.int32), device=DEV)
    sink = qqe.read_probe(a, b if two else None, waves_per_row=waves)
    torch.cuda.synchronize()
    want = _xor_rows(ha, hb) if two else _xor_rows(ha)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("waves", [1, 4])
def test_read_probe_on_bf16_rows(waves):
    g = torch.Generator(device="cpu").manual_seed(3)
    a = torch.randn((8, 151936), generator=g).to(torch.bfloat16).to(DEV)
    sink = qqe.read_probe(a, waves_per_row=waves)
    torch.cuda.synchronize()
    want = _xor_rows(a.cpu().view(torch.int16).numpy().view(np.uint16).view(np.uint32).reshape(8, -1))
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("rows", [3, 40])
def test_read_probe_records_launch_events(rows):
    """With start / stop events the probe's launch records them itself: the
    checksums are unchanged and the elapsed time is positive."""
    g = np.random.default_rng(rows)
    ha = g.integers(0, 2 ** 32, (rows, 4096), dtype=np.uint32)
    a = torch.as_tensor(ha.view(np.int32), device=DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    sink = qqe.read_probe(a, waves_per_row=4, start_event=e0, stop_event=e1)
    e1.synchronize()
    assert e0.elapsed_time(e1) > 0
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), _xor_rows(ha))
    with pytest.raises(ValueError):
        qqe.read_probe(a, start_event=torch.cuda.Event(enable_timing=True))  # never recorded: no HIP event yet
