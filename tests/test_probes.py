"""The measurement probes behind the bench's measured bounds read and write
exactly what they claim: the streaming probe's per-wavefront checksums
against a host simulation of its shares, and its written pattern; the
gather probe's checksums against the rows its index list names."""

import numpy as np
import pytest
import torch

DEV = "cuda"
pytestmark = pytest.mark.gpu


def _stream_expect(words, nchunks_w, nwaves):
    """Checksum and owner per wavefront of hswa_stream_probe: wavefront w
    reads chunks [r0, r1) of 1 KB in bursts of 8, the last burst repeating
    chunk r1 - 1 for its missing slots; it writes chunks [q0, q1)."""
    rch = words.size // 256
    chunks = words.reshape(rch, 256) if rch else words.reshape(0, 256)
    sums = np.zeros(nwaves, dtype=np.uint32)
    owner = np.zeros(nchunks_w, dtype=np.int64)
    for w in range(nwaves):
        r0, r1 = rch * w // nwaves, rch * (w + 1) // nwaves
        s = np.uint32(0)
        r = r0
        while r < r1:
            idx = np.minimum(np.arange(r, r + 8), r1 - 1)
            s ^= np.bitwise_xor.reduce(chunks[idx].ravel())
            r += min(8, r1 - r)
        sums[w] = s
        owner[nchunks_w * w // nwaves:nchunks_w * (w + 1) // nwaves] = w
    return sums, owner


@pytest.mark.parametrize("read_kb,write_kb,blocks", [
    (300, 170, 3),      # uneven shares, reads and writes interleaved
    (1024, 0, 5),       # read only
    (0, 333, 2),        # write only
    (5, 9, 4),          # fewer read chunks than wavefronts
])
def test_stream_probe(gpu_lib, read_kb, write_kb, blocks):
    g = torch.Generator().manual_seed(read_kb * 1000 + write_kb)
    src = (torch.randint(0, 2 ** 31 - 1, (read_kb * 256,), generator=g, dtype=torch.int64)
           .to(torch.int32).to(DEV)) if read_kb else None
    dst = torch.zeros(write_kb * 256, dtype=torch.int32, device=DEV) if write_kb else None
    o = gpu_lib.stream_probe(src, dst, blocks)
    torch.cuda.synchronize()
    words = (src.cpu().numpy().view(np.uint32) if read_kb else np.zeros(0, dtype=np.uint32))
    sums, owner = _stream_expect(words, write_kb, 4 * blocks)
    assert np.array_equal(o.cpu().numpy().view(np.uint32), sums)
    if write_kb:
        d = dst.cpu().numpy().view(np.uint32).reshape(write_kb, 64, 4)
        assert np.array_equal(d[:, :, 0], np.broadcast_to(np.arange(write_kb)[:, None], (write_kb, 64)))
        assert np.array_equal(d[:, :, 1], np.broadcast_to(owner[:, None], (write_kb, 64)))
        assert np.array_equal(d[:, :, 3], np.broadcast_to(np.arange(64)[None, :], (write_kb, 64)))
        assert (d[:, :, 2] < 8).all()


def test_gather_probe(gpu_lib):
    rows, nwaves, tiles = 700, 6, 3
    g = torch.Generator().manual_seed(5)
    k = torch.randint(-30000, 30000, (rows, 192), generator=g, dtype=torch.int16)
    v = torch.randint(-30000, 30000, (rows, 128), generator=g, dtype=torch.int16)
    idx = torch.randint(-5, rows + 5, (nwaves * tiles * 32,), generator=g, dtype=torch.int32)
    o = gpu_lib.gather_probe(k.view(torch.bfloat16).to(DEV), v.view(torch.bfloat16).to(DEV),
                             idx.to(DEV), tiles)
    kw = k.numpy().view(np.uint32).reshape(rows, 96)
    vw = v.numpy().view(np.uint32).reshape(rows, 64)
    cl = np.clip(idx.numpy(), 0, rows - 1).reshape(nwaves, tiles * 32)
    expect = [np.bitwise_xor.reduce(np.concatenate([kw[r].ravel(), vw[r].ravel()]))
              for r in cl]
    assert np.array_equal(o.cpu().numpy().view(np.uint32), np.array(expect, dtype=np.uint32))
