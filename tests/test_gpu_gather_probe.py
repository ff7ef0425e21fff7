"""The gather probe (a measurement helper, not a step of the method) really streams the listed
latent rows: its per-group checksum equals the one computed on the host from the same table
and row list, following the tile layout the attention kernels use."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

dev = "cuda"
GROUP = 2048


def _expected(table: np.ndarray, rows: np.ndarray, width: int) -> np.ndarray:
    """XOR per group of 2048 listed rows, over its 32-row tiles and the 256 threads l, of the
    four 32-bit words at byte 16 l of the tile: tile row r = l // (width/8), row chunk
    (l mod (width/8)) XOR swizzle(r); -1 (and the slots past the list) read row 0."""
    kch = width // 8
    words = table.view(np.uint32).reshape(table.shape[0], width // 2)
    l = np.arange(256)
    r = l // kch
    sw = (r & 7) if width == 576 else ((r & 7) << 1)
    ch = (l % kch) ^ sw
    out = []
    for g0 in range(0, len(rows), GROUP):
        ids = rows[g0:g0 + GROUP]
        nch = (len(ids) + 31) // 32
        slots = np.full(nch * 32, -1, np.int64)
        slots[:len(ids)] = ids
        slots = np.where(slots < 0, 0, slots).reshape(nch, 32)
        src = slots[:, r]                                   # [nch, 256] table rows
        cols = ch[None, :, None] * 4 + np.arange(4)[None, None, :]
        x = np.bitwise_xor.reduce(words[src[:, :, None], cols].reshape(-1))
        out.append(x)
    return np.array(out, np.uint32)


@pytest.mark.parametrize("T_kv,width,n", [(1000, 576, 5000), (700, 512, 4096), (33, 576, 31),
                                          (65536, 512, 2048 * 3 + 100)])
def test_gather_probe_checksums(T_kv, width, n):
    import sparse_attention_12_amd as dsa
    g = torch.Generator().manual_seed(T_kv + width + n)
    table = torch.randint(-32768, 32768, (T_kv, width), generator=g, dtype=torch.int32)
    table = table.to(torch.int16).view(torch.bfloat16)
    rows = torch.randint(0, T_kv, (n,), generator=g, dtype=torch.int32)
    rows[::97] = -1
    sink = dsa.gather_probe(table.to(dev), rows.to(dev))
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    exp = _expected(table.view(torch.int16).numpy().view(np.uint16), rows.numpy(), width)
    np.testing.assert_array_equal(got, exp)


def test_gather_probe_empty_list():
    import sparse_attention_12_amd as dsa
    table = torch.zeros((16, 512), dtype=torch.bfloat16, device=dev)
    rows = torch.zeros((0,), dtype=torch.int32, device=dev)
    assert dsa.gather_probe(table, rows).numel() == 0
