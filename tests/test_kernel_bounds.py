"""Host-side check of the MFMA decode kernel's row indexing: for every
(T, split size, blocks per wave step, waves) the rows its loads touch stay
below the padded token count T_pad of the device layout.

The index arithmetic below restates, in Python, what the kernel computes for
the key-operand fetches (first block of each wave in the prologue, the next
block inside the loop) and the value-operand loads of a block; the host rounds
split sizes up to 128 tokens and pads T to 128.
"""
import pytest

TOK_PAD = 128


def round_up(x, m):
    return (x + m - 1) // m * m


def touched_rows(T, split_tokens, NB, waves):
    T_pad = round_up(T, TOK_PAD)
    split = round_up(split_tokens, TOK_PAD)
    rows = set()
    n_split = (T + split - 1) // split
    for s in range(n_split):
        t0, t1 = s * split, min(T, s * split + split)
        if t0 >= t1:
            continue
        nblk = (t1 - t0 + 16 * NB - 1) // (16 * NB)
        starts = [t0 + 16 * NB * min(w, nblk - 1) for w in range(waves)]   # prologue
        starts += [t0 + 16 * NB * b for b in range(nblk)]                   # loop fetches
        for tw in starts:
            for n in range(NB):
                rows.update(range(tw + 16 * n, tw + 16 * n + 16))          # keys, values, scales
    return T_pad, rows


@pytest.mark.parametrize("NB,waves", [(1, 8), (1, 4), (2, 8)])
@pytest.mark.parametrize("split", [128, 256, 512, 1024, 2048])
def test_fetch_rows_below_T_pad(NB, waves, split):
    for T in list(range(1, 300, 7)) + [511, 512, 513, 1023, 1111, 1152, 1153, 1500, 4096, 4097]:
        T_pad, rows = touched_rows(T, split, NB, waves)
        assert max(rows) < T_pad, (T, split, NB, waves, max(rows), T_pad)


def test_old_prologue_would_overrun():
    """The prologue used to fetch block w for every wave w; with two blocks
    per step and a last split of at most 128 tokens that reads past T_pad
    (T = 1111, split 512: rows up to 1279, T_pad = 1152)."""
    T, split, NB, waves = 1111, 512, 2, 8
    T_pad = round_up(T, TOK_PAD)
    t0 = (T // split) * split
    assert t0 + 16 * NB * (waves - 1) + 16 * NB - 1 >= T_pad
    assert max(touched_rows(T, split, NB, waves)[1]) < T_pad


@pytest.mark.parametrize("H,n_split,nseq", [(32, 1, 16), (8, 4, 2), (8, 8, 3), (4, 2, 12), (2, 16, 1),
                                            (32, 3, 8)])
def test_xcd_grids_cover_every_unit_once(H, n_split, nseq):
    """The MFMA kernel's block -> (head, split, sequence) maps: every work item
    exactly once, in range, and with an XCD-aware grid all heads of one
    (sequence, split) unit on one XCD (workgroups go to XCD linear id mod 8)."""
    mode = 1 if n_split % 8 == 0 else 2 if (nseq * n_split) % 8 == 0 else 0
    if mode == 1:
        grid = (8 * H, n_split // 8, nseq)
    elif mode == 2:
        grid = (8 * H, nseq * n_split // 8, 1)
    else:
        grid = (H, n_split, nseq)
    seen, xcd_of = set(), {}
    for z in range(grid[2]):
        for y in range(grid[1]):
            for x in range(grid[0]):
                lin = x + grid[0] * (y + grid[1] * z)
                if mode == 1:
                    b, h, split = z, x >> 3, y * 8 + (x & 7)
                elif mode == 2:
                    h, u = x >> 3, y * 8 + (x & 7)
                    b, split = u // n_split, u % n_split
                else:
                    b, h, split = z, x, y
                assert 0 <= b < nseq and 0 <= h < H and 0 <= split < n_split
                seen.add((b, h, split))
                xcd_of.setdefault((b, split), set()).add(lin % 8)
    assert len(seen) == H * n_split * nseq
    if mode:
        assert all(len(v) == 1 for v in xcd_of.values())
