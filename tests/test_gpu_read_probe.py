"""The streaming-read reference kernel reads every 16-byte vector of its buffer: one
vector holding the fold's fixed value (and every other word zero) makes exactly the
thread that reads it store that value, wherever the vector sits (inside a full unrolled
round, in the ragged tail, first or last)."""
import pytest
import torch

from contextual_sparsity_amd import dejavu as dj
from helpers import DEV

pytestmark = pytest.mark.gpu

SENTINEL = 0x5EEDC0DE


@pytest.mark.parametrize("nvec,at", [(1, 0), (4096, 4095), (4 * 2**20 + 5, 2**20 + 7), (4 * 2**20 + 5, 4 * 2**20 + 4)])
def test_read_probe_reads_every_vector(nvec, at):
    buf = torch.zeros(nvec * 4, dtype=torch.int32, device=DEV)
    buf[4 * at] = SENTINEL
    out = torch.zeros(1, dtype=torch.int32, device=DEV)
    dj.dejavu_read_probe(buf, out)
    torch.cuda.synchronize()
    assert (int(out.item()) & 0xFFFFFFFF) == SENTINEL


def test_read_probe_writes_nothing_otherwise():
    buf = torch.arange(4 * 65536, dtype=torch.int32, device=DEV)
    out = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    dj.dejavu_read_probe(buf, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 7
