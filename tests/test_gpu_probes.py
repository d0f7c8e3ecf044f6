"""GPU: the two bandwidth probes through the C ABI.

pkv_copy (the kernel the HBM traffic counters are scaled by) must copy every
byte, ragged tails included; pkv_read_probe must read every byte it is given,
in address order or chunk by chunk through an index list, which its checksum
shows: the XOR of all 32-bit words read, computed here with numpy.
"""
import sys

import numpy as np
import pytest

import paged_kv_cache_152_amd as pkv

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def xor_words(raw: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(raw.view(np.uint32))) if raw.size else 0


# sizes in bytes: one 16-byte word, less than one workgroup run, a ragged run,
# several runs per workgroup of the largest grid (2048 workgroups for the copy)
SIZES = [16, 4096, 16 * 1024 + 48, (2048 * 16 * 1024) * 3 + 16 * 1000]


@pytest.mark.parametrize("nbytes", SIZES)
def test_copy_probe_copies_every_byte(nbytes):
    say(f"[test] pkv_copy {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    raw = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(raw).cuda()
    dst = torch.full_like(src, 0xA5)
    pkv.copy(dst, src)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), raw)


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("nbytes", SIZES)
def test_read_probe_checksum_covers_every_word(nbytes, nontemporal):
    say(f"[test] pkv_read_probe {nbytes} bytes nontemporal={nontemporal}")
    rng = np.random.default_rng(nbytes + 1)
    raw = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(raw).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.read_probe(src, sink, nontemporal)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    assert got == xor_words(raw)
    # a second pass XORs the same checksum in again
    pkv.read_probe(src, sink, nontemporal)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("chunk_bytes,n_chunks,n_order", [(4096, 300, 1000), (32768, 40, 77), (4096, 5000, 5000),
                                                         (1 << 20, 3, 5)])
def test_gather_read_probe_checksum(chunk_bytes, n_chunks, n_order, nontemporal):
    say(f"[test] pkv_read_probe gathered: {n_order} of {n_chunks} chunks of {chunk_bytes} B, nontemporal={nontemporal}")
    rng = np.random.default_rng(chunk_bytes + n_order)
    raw = rng.integers(0, 256, chunk_bytes * n_chunks, dtype=np.uint8)
    # indices with repeats (which cancel in the XOR) and entries outside the buffer (skipped)
    order = rng.integers(-3, n_chunks + 3, n_order).astype(np.int32)
    chunks = raw.reshape(n_chunks, chunk_bytes)
    want = 0
    for c in order:
        if 0 <= c < n_chunks:
            want ^= xor_words(chunks[c])
    src = torch.from_numpy(raw).cuda()
    dorder = torch.from_numpy(order).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.read_probe(src, sink, nontemporal, order=dorder, chunk_bytes=chunk_bytes)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want


def test_read_probe_empty_and_bad_arguments():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    pkv.read_probe(empty, sink, True)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    odd = torch.zeros(24, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(odd, sink, False)
    buf = torch.zeros(3 * 4096, dtype=torch.uint8, device="cuda")
    order = torch.zeros(4, dtype=torch.int32, device="cuda")
    for chunk_bytes in (0, 2048, 3 * 4096, 8192):        # not 4096 x 2^k, or not dividing the buffer
        with pytest.raises(pkv.PagedKVError):
            pkv.read_probe(buf, sink, True, order=order, chunk_bytes=chunk_bytes)
    pkv.read_probe(buf, sink, True, order=order[:0], chunk_bytes=4096)   # empty list: nothing read
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
