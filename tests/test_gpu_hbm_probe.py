"""The streaming-read probe behind roofline.achievable reads every byte it is
given (GPU, through the C ABI).

The probe folds what each thread reads with XOR and writes the fold to its
sink only when it equals a fixed constant.  A zero buffer with one 16-byte
unit holding that constant therefore marks the sink exactly when the unit
was read: placed at the first and last unit, on both sides of a workgroup's
32 KiB chunk and of a 4 KiB round, and at the ragged end of the buffer, it
shows that no part of the buffer is skipped.  A zero buffer never marks it."""
import numpy as np
import pytest
import torch

from tests.gpu_util import announce, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8

MARK = np.uint32(0x9E3779B9).view(np.int32).item()   # the probe's constant, as int32 bits


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def probe_marks(units: int, pos) -> bool:
    buf = torch.zeros(units * 4, dtype=torch.int32, device="cuda:0")
    if pos is not None:
        buf[4 * pos] = MARK
    sink = torch.zeros(w8.HBM_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda:0")
    w8.hbm_read_probe(buf, sink=sink)
    torch.cuda.synchronize()
    return int(sink[0].item()) == MARK


@pytest.mark.parametrize("units", [1, 255, 2048 * 3 + 5, 2048 * 40 + 2047])
def test_probe_reads_every_unit(units):
    announce(f"hbm_read_probe coverage units={units}")
    assert not probe_marks(units, None)
    positions = sorted({0, units - 1, min(255, units - 1), min(256, units - 1),
                        min(2047, units - 1), min(2048, units - 1), units // 2,
                        max(0, units - 2049)})
    for p in positions:
        assert probe_marks(units, p), f"unit {p} of {units} not read"


def test_probe_reads_the_last_unit_of_a_large_buffer():
    units = (622_329_856 + 16 * 3) // 16      # the LM head's bytes and a ragged tail
    announce(f"hbm_read_probe last unit of {units * 16} bytes")
    assert probe_marks(units, units - 1)
    assert probe_marks(units, units // 3)
