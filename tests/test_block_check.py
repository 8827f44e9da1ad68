"""fs_check_block_tables, the opt-in host check that one call's requests
write distinct cache blocks (runs on the CPU: no store, no GPU).  Pinned by
hand cases and by a brute-force reference on random tables."""

import numpy as np
import pytest

from kv_cache_injection_amd import fs


def _reference(bt, sp, nt, bs, nb):
    """Brute force: (status, conflict) with the documented conflict order."""
    uses = []
    for b in range(bt.shape[0]):
        s, L = int(sp[b]), int(nt[b])
        if L <= 0:
            continue
        if s < 0:
            return fs.FS_E_BLOCKTABLE, [b, -1, -1, -1]
        last = (s + L - 1) // bs
        if last >= bt.shape[1]:
            return fs.FS_E_BLOCKTABLE, [b, last, -1, -1]
        for j in range(s // bs, last + 1):
            i = int(bt[b, j])
            if i < 0 or i >= nb:
                return fs.FS_E_BLOCKTABLE, [b, j, i, -1]
            uses.append((i, b, j))
    seen = {}
    for i, b, j in sorted(uses, key=lambda u: u[0]):      # stable: (b, j) order within an id
        if i in seen:
            return fs.FS_E_BLOCKTABLE, [b, j, i, seen[i]]
        seen[i] = b
    return fs.FS_OK, [-1, -1, -1, -1]


def _check(bt, sp, nt, bs, nb):
    try:
        fs.fs_check_block_tables(bt, sp, nt, bs, nb)
        return fs.FS_OK, [-1, -1, -1, -1]
    except fs.FsError as e:
        return e.status, e.conflict


def test_hand_cases():
    bt = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], np.int32)
    # request 0 writes positions 10..40 (blocks 0..2 of 16), request 1 positions 0..15 (block 0)
    assert _check(bt, [10, 0], [31, 16], 16, 8) == (fs.FS_OK, [-1, -1, -1, -1])
    bt2 = bt.copy()
    bt2[1, 0] = 2                          # request 1's block 0 is request 0's block 2
    assert _check(bt2, [10, 0], [31, 16], 16, 8) == (fs.FS_E_BLOCKTABLE, [1, 0, 2, 0])
    # the aliased block is not written by request 0 when its segment is shorter
    assert _check(bt2, [10, 0], [20, 16], 16, 8) == (fs.FS_OK, [-1, -1, -1, -1])
    bt3 = bt.copy()
    bt3[0, 2] = 0                          # one request naming a block twice
    assert _check(bt3, [10, 0], [31, 0], 16, 8) == (fs.FS_E_BLOCKTABLE, [0, 2, 0, 0])
    assert _check(bt, [10, 0], [31, 16], 16, 4) == (fs.FS_E_BLOCKTABLE, [1, 0, 4, -1])  # id 4 out of range
    assert _check(bt, [10, 0], [31, 16], 16, 5) == (fs.FS_OK, [-1, -1, -1, -1])          # ids 5..7 unused
    assert _check(bt, [60, 0], [10, 0], 16, 8) == (fs.FS_E_BLOCKTABLE, [0, 4, -1, -1])  # beyond the table
    assert _check(bt, [0, 0], [0, 0], 16, 8) == (fs.FS_OK, [-1, -1, -1, -1])           # nothing written
    with pytest.raises(fs.FsError) as e:
        fs.fs_check_block_tables(bt, [0, 0], [1, 1], 12, 8)                   # not a power of two
    assert e.value.status == fs.FS_E_ARG


def test_out_of_range_id_is_named():
    bt = np.array([[0, 9]], np.int32)
    assert _check(bt, [0], [32], 16, 8) == (fs.FS_E_BLOCKTABLE, [0, 1, 9, -1])


@pytest.mark.parametrize("seed", range(40))
def test_random_tables_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 12))
    bs = int(rng.choice([1, 2, 4, 16, 64]))
    mb = int(rng.integers(1, 20))
    nb = int(rng.integers(1, batch * mb + 5))
    if rng.random() < 0.5:                 # distinct ids (a valid layout) ...
        ids = rng.permutation(max(nb, batch * mb))[: batch * mb] % nb
    else:                                  # ... or ids drawn with repeats
        ids = rng.integers(0, nb, batch * mb)
    bt = ids.reshape(batch, mb).astype(np.int32)
    if rng.random() < 0.2:
        bt[rng.integers(batch), rng.integers(mb)] = int(rng.choice([-1, nb]))
    sp = rng.integers(0, mb * bs, batch).astype(np.int32)
    nt = rng.integers(0, mb * bs, batch).astype(np.int32)
    if rng.random() < 0.5:
        nt = np.minimum(nt, mb * bs - sp).astype(np.int32)              # mostly within the table
    assert _check(bt, sp, nt, bs, nb) == _reference(bt, sp, nt, bs, nb)
