"""The streaming-read probe (a measurement aid beside the decode indexer) reads
every tile it is given: a word planted in a buffer of zeros so that one lane's
XOR fold equals the probe's sink pattern must reach the sink, whatever tile and
launch shape holds it; a buffer of zeros leaves the sink alone."""
import sys

import pytest
import torch

import dsa_sparse_attention_lightning_amd as dsa

pytestmark = pytest.mark.gpu

PATTERN = 0x9E3779B9 - (1 << 32)  # the fold value that is stored, as an int32
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("form", ["tiles", "stride"])
@pytest.mark.parametrize("tiles,workgroups,plant_tile",
                         [(1, 1, 0), (17, 3, 16), (40, 256, 39), (17417, 256, 12345),
                          (17417, 2048, 17416)])
def test_probe_reads_every_tile(form, tiles, workgroups, plant_tile):
    say(f"stream probe {form}: {tiles} tiles, {workgroups} workgroups, word in tile {plant_tile}")
    buf = torch.zeros(tiles * 2048, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.probe_stream_read(buf, sink, workgroups, form)
    torch.cuda.synchronize()
    assert sink.item() == 0
    # One 32-bit word: only the lane that loads it folds to the pattern.
    buf[plant_tile * 2048 + 37 * 4 + 1] = PATTERN
    dsa.probe_stream_read(buf, sink, workgroups, form)
    torch.cuda.synchronize()
    assert sink.item() == PATTERN


def test_probe_rejects_partial_tiles():
    buf = torch.zeros(1000, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(Exception, match="8192"):
        dsa.probe_stream_read(buf, sink, 4, "tiles")
