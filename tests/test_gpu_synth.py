"""The compute-free row read that the benchmark times beside the gather (a bandwidth
reference, not the product path): it must read exactly the rows the bags name."""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_rows,words,n_bags,bag", [
    (1000, 1024, 37, 128),   # 4 KiB rows: one bag per block, 16 rows in flight
    (300, 512, 9, 19),       # 2 KiB rows: two bags per block; a ragged tail after 16 rows
    (64, 16, 70, 5),         # 64-byte rows: 64 bags per block; no 16-row round
    (50, 1280, 3, 17),       # 5 KiB rows: two column blocks, the second partly idle
])
def test_row_read_xors_the_rows_of_each_bag(n_rows, words, n_bags, bag):
    from synth import device as SD
    say(f"row_read n_rows={n_rows} row_bytes={4 * words} bags={n_bags}x{bag}")
    g = torch.Generator().manual_seed(n_rows * 31 + bag)
    table = torch.randint(-2**31, 2**31 - 1, (n_rows, words), generator=g, dtype=torch.int64).to(torch.int32)
    idx = torch.randint(0, n_rows, (n_bags, bag), generator=g, dtype=torch.int64).to(torch.int32)
    idx[0, 0] = -1          # out of range: reads row 0
    idx[-1, -1] = n_rows    # out of range: reads row 0
    out = torch.full((n_bags, words), 7, dtype=torch.int32, device="cuda")
    SD.row_read(table.cuda(), idx.cuda(), out)
    torch.cuda.synchronize()
    t = table.numpy().view(np.uint32)
    i = idx.numpy().astype(np.int64)
    i = np.where((i >= 0) & (i < n_rows), i, 0)
    want = np.bitwise_xor.reduce(t[i], axis=1)
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
