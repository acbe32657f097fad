"""The two measurement probes on the GPU, through the C ABI, checked against
values fixed by their definitions (include/hs2.h):

  * hs2_probe_mfma: without operands every thread's sink word is
    128 * iters * one^2 exactly (A all `one`, B all `one`/16, 8 chains of 16
    accumulators a lane); with small-integer operands it is 8 * iters times
    the sum of the lane's 16 entries of the 32 x 32 product D = A B, laid out
    as the 32x32x16 instruction holds it (lane l: column l % 32, entry i at
    row 8 (i / 4) + 4 (l / 32) + i % 4), all exact in fp32.
  * hs2_probe_gather: the XOR of all sink words equals the XOR of every
    32-bit word of every gathered row (and of its scale, when given). XOR is
    order-free, so this holds however the kernel deals rows to threads, as
    long as no row is read twice: n_idx is a multiple of the kernel's step
    (16 rows x 8 in flight for 256-byte rows, 32 x 8 for 128-byte rows).
    An index outside [0, n_rows) reads row 0.
  * hs2_probe_stream: the XOR of all sink words equals the XOR of every
    32-bit word of src (each 4 KiB chunk read once), and dst chunk
    g + G w holds a copy of src chunk g + G (R (w + 1) - 1) where that chunk
    exists (G workgroups, R reads per write), the rest of dst and a guard band
    past it untouched.
"""
import sys

import numpy as np
import pytest
import torch

import token_level_top_amd as hs2

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("wps", [1, 2])
@pytest.mark.parametrize("n_blocks,iters,one", [(3, 7, 1.0), (300, 50, 0.5), (256, 1000, 2.0)])
def test_probe_mfma_exact(wps, n_blocks, iters, one):
    say(f"probe_mfma wps={wps} n_blocks={n_blocks} iters={iters} one={one}")
    sink = hs2.probe_mfma(wps, n_blocks, iters, one)
    torch.cuda.synchronize()
    want = 128.0 * iters * one * one
    got = sink.cpu().numpy()
    assert got.shape == (n_blocks * 256 * wps,)
    assert np.all(got == np.float32(want)), (got.min(), got.max(), want)


@pytest.mark.parametrize("wps", [1, 2])
def test_probe_mfma_operands_exact(wps):
    say(f"probe_mfma with operands wps={wps}")
    g = torch.Generator().manual_seed(9)
    ops = torch.randint(-2, 3, (64, 16), generator=g).to(torch.bfloat16)
    n_blocks, iters = 5, 50
    sink = hs2.probe_mfma(wps, n_blocks, iters, 0.0, ops.cuda())
    torch.cuda.synchronize()
    o = ops.float().numpy()
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for l in range(64):
        A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = o[l, :8]
        Bm[8 * (l // 32):8 * (l // 32) + 8, l % 32] = o[l, 8:]
    D = A @ Bm
    lane_sum = np.array([sum(D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] for i in range(16)) for l in range(64)])
    want = np.tile(8 * iters * lane_sum, n_blocks * 4 * wps).astype(np.float32)
    got = sink.cpu().numpy()
    assert np.array_equal(got, want), np.abs(got - want).max()


@pytest.mark.parametrize("row_bytes,with_scale", [(256, False), (128, True), (128, False)])
def test_probe_gather_xor(row_bytes, with_scale):
    say(f"probe_gather row_bytes={row_bytes} scale={with_scale}")
    g = torch.Generator().manual_seed(5)
    n_rows, n_idx = 5000, 4096 * 3
    src = torch.randint(0, 256, (n_rows, row_bytes), dtype=torch.uint8, generator=g)
    scale = torch.rand(n_rows, generator=g) if with_scale else None
    idx = torch.randint(-50, n_rows + 50, (n_idx,), dtype=torch.int32, generator=g)  # some out of range
    sink = torch.zeros(524288, dtype=torch.int32, device="cuda")  # words past the grid stay zero
    hs2.probe_gather(src.cuda(), idx.cuda(), scale.cuda() if with_scale else None, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    rows = np.where((idx.numpy() >= 0) & (idx.numpy() < n_rows), idx.numpy(), 0)
    words = src.numpy().view(np.uint32)[rows]
    want = np.bitwise_xor.reduce(words.reshape(-1))
    if with_scale:
        want ^= np.bitwise_xor.reduce(scale.numpy().view(np.uint32)[rows])
    assert got == want, (hex(got), hex(want))


@pytest.mark.parametrize("n_chunks,n_dst,n_blocks,rpw", [(16387, 2100, 300, 8), (1000, 1200, 64, 1),
                                                         (5000, 100, 256, 4), (3001, 700, 7, 2), (777, 0, 100, 0)])
def test_probe_stream_exact(n_chunks, n_dst, n_blocks, rpw):
    say(f"probe_stream chunks={n_chunks} dst={n_dst} blocks={n_blocks} rpw={rpw}")
    g = torch.Generator().manual_seed(n_chunks + rpw)
    src = torch.randint(0, 256, (n_chunks * 4096,), dtype=torch.uint8, generator=g)
    guard = 16
    dst = torch.full(((n_dst + guard) * 4096,), 0xA5, dtype=torch.uint8, device="cuda") if rpw else None
    src_d = src.cuda()
    sink = torch.empty(n_blocks * 256, dtype=torch.int32, device="cuda")
    if rpw:
        rc = hs2.lib().hs2_probe_stream(src_d.data_ptr(), src_d.numel(), dst.data_ptr(), n_dst * 4096, rpw, n_blocks,
                                        sink.data_ptr(), sink.numel(), None)
    else:
        rc = hs2.lib().hs2_probe_stream(src_d.data_ptr(), src_d.numel(), None, 0, 0, n_blocks, sink.data_ptr(),
                                        sink.numel(), None)
    assert rc == hs2.HS2_OK
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want, f"XOR of sink {got:#x} != XOR of src {want:#x}"
    if rpw:
        d = dst.cpu().numpy().reshape(-1, 4096)
        sc = src.numpy().reshape(-1, 4096)
        dc = np.arange(n_dst)
        from_chunk = dc % n_blocks + n_blocks * (rpw * (dc // n_blocks + 1) - 1)
        written = from_chunk < n_chunks
        assert np.array_equal(d[:n_dst][written], sc[from_chunk[written]]), "copied chunks differ"
        assert (d[:n_dst][~written] == 0xA5).all(), "a chunk with no source chunk was written"
        assert (d[n_dst:] == 0xA5).all(), "guard band past dst_bytes written"
        say(f"  {int(written.sum())} of {n_dst} dst chunks copied, guard band intact")
