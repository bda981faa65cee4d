"""The stream-read probe reads every 16-byte piece of its buffer: a lane
stores the magic word only when the xor of the words it loaded equals it,
so a zero buffer leaves the sink untouched and a single piece holding the
magic word, wherever it sits (first piece, last piece of a ragged tail,
the middle of a large buffer), makes the sink take it."""
import pytest
import torch

import query_aware_kv_amd as qa

import gpu_cases as C

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
UNTOUCHED = 0x12345678


def _probe(words: torch.Tensor) -> int:
    sink = torch.full((1,), UNTOUCHED, dtype=torch.int32, device="cuda")
    qa.quest_stream_read_probe(words, sink)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("pieces", [1, 7, 1024 * 5 + 7, (64 << 20) // 16 + 3])
def test_probe_reads_every_piece(pieces):
    C.say(f"[case] stream read probe, {pieces} pieces of 16 bytes")
    words = torch.zeros(pieces * 4, dtype=torch.int32, device="cuda")
    assert _probe(words) == UNTOUCHED
    magic = MAGIC - (1 << 32)  # the same 32 bits as an int32
    for at in sorted({0, pieces // 2, pieces - 1}):
        words.zero_()
        words[4 * at + 1] = magic
        assert _probe(words) == MAGIC, at
