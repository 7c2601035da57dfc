"""The measurement probe (include/moe_probe.h) moves the bytes it claims:
every written row is the XOR of its item's read rows, contiguous or through
row-index arrays, and rows outside the mapping stay untouched."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("items,row_bytes,reads,writes,perm_side", [
    (37, 2064, 1, 8, None), (37, 2064, 1, 8, "dst"), (29, 14336, 9, 1, None),
    (29, 14336, 9, 1, "src"), (5, 16, 16, 16, "both"),
])
def test_stream_mix_moves_the_rows(items, row_bytes, reads, writes, perm_side):
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(items + reads)
    n_src, n_dst = items * reads + 3, items * writes + 5
    words = row_bytes // 4
    src_np = rng.integers(0, 2**32, size=(n_src, words), dtype=np.uint64).astype(np.uint32)
    src_rows = dst_rows = None
    s_idx = np.arange(items * reads).reshape(items, reads)
    d_idx = np.arange(items * writes).reshape(items, writes)
    if perm_side in ("src", "both"):
        s_idx = rng.permutation(n_src)[:items * reads].reshape(items, reads)
        src_rows = torch.from_numpy(s_idx.astype(np.int32).ravel()).cuda()
    if perm_side in ("dst", "both"):
        d_idx = rng.permutation(n_dst)[:items * writes].reshape(items, writes)
        dst_rows = torch.from_numpy(d_idx.astype(np.int32).ravel()).cuda()
    src = torch.from_numpy(src_np.view(np.int32)).cuda()
    dst = torch.full((n_dst, words), -1, dtype=torch.int32, device="cuda")
    moe.moe_probe_stream_mix(src, dst, items, reads, writes, src_rows, dst_rows)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    ref = np.full((n_dst, words), 0xFFFFFFFF, np.uint32)
    for i in range(items):
        acc = np.bitwise_xor.reduce(src_np[s_idx[i]], axis=0)
        ref[d_idx[i]] = acc
    np.testing.assert_array_equal(got, ref)
