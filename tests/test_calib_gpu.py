"""The HBM calibration kernels move what they say they move (GPU).  They are measurement
helpers, not part of the model, so torch's own tensor operations check them."""
import numpy as np
import pytest
import torch

import embedding_lookup_feature_amd as elf
from embedding_lookup_feature_amd import embcore as ec

pytestmark = pytest.mark.gpu
DEV = "cuda"


def words(n, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(-2**31, 2**31 - 1, (n,), generator=g, device=DEV, dtype=torch.int32)


POLICIES = [0, ec.EL_CALIB_NT_LOADS, ec.EL_CALIB_NT_STORES, ec.EL_CALIB_NT_LOADS | ec.EL_CALIB_NT_STORES]


@pytest.mark.parametrize("policy", POLICIES)
def test_copy_write_and_read3_write1_move_the_right_bytes(policy):
    nbytes = 3 << 20
    src = words(nbytes // 4, 1)
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    elf.hbm_calib(ec.EL_CALIB_COPY | policy, src, dst, nbytes)  # half the traffic read, half written
    torch.cuda.synchronize()
    half = nbytes // 8
    assert torch.equal(dst[:half], src[:half]) and torch.count_nonzero(dst[half:]) == 0
    dst.zero_()
    elf.hbm_calib(ec.EL_CALIB_READ3_WRITE1 | policy, src, dst, nbytes)
    torch.cuda.synchronize()
    m = nbytes // 64  # output vectors; three input streams of m vectors each
    sv = src.view(-1, 4)
    assert torch.equal(dst.view(-1, 4)[:m], sv[:m] ^ sv[m:2 * m] ^ sv[2 * m:3 * m])
    assert torch.count_nonzero(dst.view(-1, 4)[m:]) == 0
    dst.zero_()
    elf.hbm_calib(ec.EL_CALIB_WRITE | policy, None, dst, nbytes)
    torch.cuda.synchronize()
    v = dst.view(-1, 4)
    assert torch.equal(v[:, 0], torch.arange(v.shape[0], device=DEV, dtype=torch.int32))
    assert torch.equal(v[:, 1:], torch.tensor([1, 2, 3], device=DEV, dtype=torch.int32).expand(v.shape[0], 3))


@pytest.mark.parametrize("policy", [0, ec.EL_CALIB_NT_LOADS])
def test_read_leaves_per_thread_xors(policy):
    n = (1 << 20) + 16 * 777  # 4 MiB of int32 and a partial chunk
    src = words(n, 2)
    sink = torch.zeros(2 << 20, dtype=torch.int32, device=DEV)  # 8 MiB: one 16-byte slot per thread
    elf.hbm_calib(ec.EL_CALIB_READ | policy, src, sink, 4 * n)
    torch.cuda.synchronize()
    # the xor of all the per-thread xors is the xor of the whole buffer, word by word
    got = sink.view(-1, 4).cpu().numpy()
    ref = src.view(-1, 4).cpu().numpy()
    assert np.array_equal(np.bitwise_xor.reduce(got, axis=0), np.bitwise_xor.reduce(ref, axis=0))


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("row_bytes", [16, 128, 256, 512, 1024])
def test_gather_copies_the_indexed_rows(row_bytes, policy):
    rows = 5000
    table = words(rows * row_bytes // 4, 3).view(rows, row_bytes // 4)
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    idx = torch.randint(0, rows, (7777,), generator=g, device=DEV, dtype=torch.int32)
    dst = torch.zeros((idx.numel(), row_bytes // 4), dtype=torch.int32, device=DEV)
    elf.hbm_calib(ec.EL_CALIB_GATHER | policy, table, dst, 0, idx=idx, row_bytes=row_bytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, table.index_select(0, idx.long()))
    if row_bytes >= 32:  # the first half of every row only
        half = torch.zeros((idx.numel(), row_bytes // 8), dtype=torch.int32, device=DEV)
        elf.hbm_calib(ec.EL_CALIB_GATHER | policy, table, half, row_bytes // 2, idx=idx, row_bytes=row_bytes)
        torch.cuda.synchronize()
        assert torch.equal(half, table.index_select(0, idx.long())[:, :row_bytes // 8])
    sink = torch.zeros(2 << 20, dtype=torch.int32, device=DEV)  # one 16-byte slot per thread
    elf.hbm_calib(ec.EL_CALIB_GATHER_READ | (policy & ec.EL_CALIB_NT_LOADS), table, sink, 0, idx=idx,
                  row_bytes=row_bytes)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.view(-1, 4).cpu().numpy(), axis=0)
    rows = table.index_select(0, idx.long()).view(-1, 4).cpu().numpy()
    assert np.array_equal(got, np.bitwise_xor.reduce(rows, axis=0))
