"""GPU: attn_decode_check_tables counts exactly the out-of-range lengths and used
block-table entries that include/attn.h defines, against a plain Python count of the
same definition (slots past a sequence's length are not read and not counted)."""
import numpy as np
import pytest
import torch

from exact_io_aware_prefill_amd import workloads as W
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def expected_count(bt, lens, page, max_blocks, num_blocks, appended):
    """The header's definition, written out element by element."""
    cap = max_blocks * page
    bad = 0
    for b, L in enumerate(lens):
        need = int(L) + appended
        if L < 0 or need > cap:
            bad += 1
        if bt is not None:
            used = min(max(need, 0), cap)
            for j in range(max_blocks):
                if j * page < used and not (0 <= int(bt[b][j]) < num_blocks):
                    bad += 1
    return bad


def run(attn, bt, lens, page, max_blocks, num_blocks, appended):
    out = torch.full((1,), 77, dtype=torch.int32, device="cuda")  # must be overwritten
    attn.attn_decode_check_tables(None if bt is None else torch.as_tensor(bt, dtype=torch.int32).cuda(),
                                  torch.as_tensor(lens, dtype=torch.int32).cuda(), page, max_blocks, num_blocks,
                                  appended, out)
    torch.cuda.synchronize()
    return int(out.item())


def test_valid_paged_batch_has_no_bad_entries(attn):
    y = W.decode_paged_inputs(31, 32, 8, 4, 64, 16, 1024, 32768)  # the batched layout, smaller heads
    num_blocks = y.k_cache.shape[0]
    got = run(attn, y.block_table.numpy(), y.seq_lens.numpy(), y.page_size, y.max_blocks, num_blocks, False)
    say("valid paged batch: bad =", got)
    assert got == 0
    # appending one token to each sequence: only sequences already at capacity overflow
    lens = y.seq_lens.numpy()
    exp = expected_count(y.block_table.numpy(), lens, y.page_size, y.max_blocks, num_blocks, 1)
    assert run(attn, y.block_table.numpy(), lens, y.page_size, y.max_blocks, num_blocks, True) == exp


def test_planted_errors_are_counted_exactly(attn):
    page, mb, nb = 16, 6, 40
    rng = np.random.default_rng(32)
    lens = np.array([45, 0, 96, 17, -5, 97, 16], dtype=np.int32)  # -5 < 0; 97 > 6 * 16
    bt = rng.integers(0, nb, size=(len(lens), mb)).astype(np.int32)
    bt[0, 3:] = -1         # unused slots of a 45-token sequence: not read, not counted
    bt[0, 2] = nb          # used slot out of range
    bt[1, :] = 12345       # empty sequence: nothing read
    bt[2, 5] = -7          # last used slot of a full sequence
    bt[3, 1] = nb + 100    # token 16 of a 17-token sequence sits in slot 1
    bt[6, 1] = -1          # a 16-token sequence uses slot 0 only ...
    exp = expected_count(bt, lens, page, mb, nb, 0)
    got = run(attn, bt, lens, page, mb, nb, False)
    say("planted: expected", exp, "got", got)
    assert exp == 5 and got == exp  # sequences 0, 2, 3 (slots) and 4, 5 (lengths)
    # ... but with an append its token 16 lands in slot 1; the empty sequence's slot 0
    # (12345) is read; and the 96-token sequence overflows
    exp1 = expected_count(bt, lens, page, mb, nb, 1)
    assert exp1 == exp + 3 and run(attn, bt, lens, page, mb, nb, True) == exp1


def test_contiguous_cache_checks_lengths_only(attn):
    lens = np.array([0, 64, 65, -1, 64], dtype=np.int32)
    assert run(attn, None, lens, 16, 4, 0, False) == 2
    assert run(attn, None, lens, 16, 4, 0, True) == 4


def test_empty_batch_writes_zero(attn):
    assert run(attn, np.zeros((0, 4), np.int32), np.zeros((0,), np.int32), 16, 4, 8, False) == 0


def test_large_random_tables(attn):
    rng = np.random.default_rng(33)
    B, page, mb, nb = 700, 16, 300, 100000
    lens = rng.integers(-3, mb * page + 5, size=B).astype(np.int32)
    bt = rng.integers(0, nb, size=(B, mb)).astype(np.int32)
    mask = rng.random(size=(B, mb)) < 0.01
    bt[mask] = rng.choice(np.array([-1, nb, nb + 7, -(2 ** 31)], dtype=np.int64), size=int(mask.sum())).astype(np.int32)
    # vectorised form of the same definition for this size
    cap = mb * page
    need = lens.astype(np.int64)
    bad_len = int(((lens < 0) | (need > cap)).sum())
    used = np.clip(need, 0, cap)
    slot_used = (np.arange(mb)[None, :] * page) < used[:, None]
    bad_slot = int((slot_used & ((bt < 0) | (bt >= nb))).sum())
    got = run(attn, bt, lens, page, mb, nb, False)
    say("random tables: expected", bad_len + bad_slot, "got", got)
    assert got == bad_len + bad_slot
