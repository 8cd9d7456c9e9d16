"""The calibration kernels on the GPU, through the C ABI.

dec_probe_read must read every byte of its range, and only those: with the buffer all
zeros and one word set to the magic value, exactly the lane that loads that word sees its
32 words XOR to the magic and writes its global lane index (wavefront w reads bytes
[8192 w, 8192 w + 8192), lane l the 16 bytes at 16 l + 1024 u, u = 0..7), which this test
computes from the position alone.  Two magic words in one lane cancel, so nothing is
written; a magic word just past the range is never read.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from tests import hip_path as hp  # noqa: E402

MAGIC = 0x9E3779B9
UNSET = 0x7FFFFFF0


def _lane_of(byte_pos):
    wave, off = divmod(byte_pos, 8192)
    return wave * 64 + (off % 1024) // 16


def _run(nbytes, words, extra=64):
    host = np.zeros((nbytes + extra) // 4, np.uint32)
    for p in words:
        host[p // 4] = MAGIC
    buf = torch.from_numpy(host.view(np.int32)).to(hp.DEV)
    sink = torch.full((1,), UNSET, dtype=torch.int32, device=hp.DEV)
    dec.dec_probe_read(buf, nbytes, sink)
    return int(sink.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("nbytes", [16, 1024, 8192, 8192 * 4 * 3 + 48, 4 << 20])
def test_probe_reads_every_word_of_its_range(nbytes):
    print(f"[probe] bytes={nbytes}", flush=True)
    positions = sorted({0, 12, nbytes - 4, (nbytes // 2) & ~3, (nbytes // 3) & ~3})
    for p in positions:
        assert _run(nbytes, [p]) == _lane_of(p), p


def test_two_magic_words_in_one_lane_cancel_and_nothing_past_the_range_is_read():
    assert _run(8192 * 8, [5 * 8192 + 3 * 1024 + 16 * 9, 5 * 8192 + 6 * 1024 + 16 * 9 + 8]) == UNSET
    assert _run(8192 * 2 + 32, [8192 * 2 + 32]) == UNSET      # the first word past the end
    assert _run(8192 * 2 + 32, [8192 * 2 + 28]) == _lane_of(8192 * 2 + 28)


def test_empty_kernel_runs():
    dec.dec_probe_empty()
    torch.cuda.synchronize()


def test_clock_readings_bracket_the_work_between_them():
    # dec_probe_clock before and after a 1 GiB streaming read: on every XCD that recorded
    # both readings the difference is the read's duration (HIP events around the same work
    # bracket it, with the clocks' 10 ns ticks), and the readings fill at least 4 XCD slots
    n = 1 << 30
    buf = torch.zeros(n, dtype=torch.uint8, device=hp.DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=hp.DEV)
    c0 = torch.zeros(16, dtype=torch.int64, device=hp.DEV)
    c1 = torch.zeros(16, dtype=torch.int64, device=hp.DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dec.dec_probe_read(buf, n, sink)               # warm
    torch.cuda.synchronize()
    e0.record()
    dec.dec_probe_clock(c0)
    dec.dec_probe_read(buf, n, sink)
    dec.dec_probe_clock(c1)
    e1.record()
    torch.cuda.synchronize()
    a, b = c0.cpu().numpy(), c1.cpu().numpy()
    both = (a > 0) & (b > 0)
    print(f"[clock] slots {np.nonzero(both)[0].tolist()}", flush=True)
    assert both.sum() >= 4
    ev_us = e0.elapsed_time(e1) * 1e3
    for x in np.nonzero(both)[0]:
        us = (int(b[x]) - int(a[x])) * 0.01
        assert 0.5 * ev_us - 20 <= us <= ev_us + 1, (int(x), us, ev_us)
