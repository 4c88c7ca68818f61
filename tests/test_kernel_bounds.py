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
