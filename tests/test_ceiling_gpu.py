"""The measurement kernels: the streaming-read ceiling reads every 16-byte piece of its buffer, and
both entry points run and reject bad arguments."""
import numpy as np
import pytest
import torch

from weight_only_bit_w4_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"
# The read kernel folds each lane's pieces by XOR and writes its sink word only when the fold is
# this value; a buffer of zeros with one piece [MAGIC, 0, 0, 0] makes exactly the lane that reads
# that piece write it.
MAGIC = 0x9E3779B9


@pytest.mark.parametrize("pieces", [1, 63, 2047, 2048 * 3 + 1, 2293760, 4 * 2**20 + 5])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_stream_read_reads_every_piece(pieces, where):
    buf = torch.zeros(pieces * 4, dtype=torch.int32, device=DEV)
    p = {"first": 0, "middle": pieces // 2, "last": pieces - 1}[where]
    buf[4 * p] = int(np.array(MAGIC, dtype=np.uint32).view(np.int32))
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    B.w4_ceiling_stream_read(buf, sink)
    torch.cuda.synchronize()
    hits = (sink.cpu().numpy().view(np.uint32) == MAGIC).sum()
    assert hits == 1, f"piece {p} of {pieces}: {hits} sink words written"


def test_stream_read_zeros_write_nothing():
    buf = torch.zeros(2048 * 16, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    B.w4_ceiling_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0


def test_ceilings_run_and_reject_bad_arguments():
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    B.w4_ceiling_mfma(sink, 16)
    torch.cuda.synchronize()
    with pytest.raises(B.W4Error):
        B.w4_ceiling_mfma(sink, 0)
    odd = torch.zeros(5, dtype=torch.int16, device=DEV)  # 10 bytes: not a multiple of 16
    with pytest.raises(B.W4Error):
        B.w4_ceiling_stream_read(odd, sink)
