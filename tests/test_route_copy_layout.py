"""CPU replay of the large-batch router kernel's direct-to-LDS copies.

Each copy moves 8 rows x 2 k-steps (128 contiguous bytes of each row): copy
lane l fetches piece (l%8) ^ (l/8) of row l/8 into slot l, and the MFMA
fragment of lane L (row L%16 of a 16-row tile, k offset 8*(L/16)) is read
from slot (L%8)*8 + (((s%2)*4 + L/16) ^ (L%8)) of its 8-row half. These
tests recompute both sides from the same formulas as router_logits_wide_kernel
and check that every fragment element a lane reads is the element the
16-token / 16-expert MFMA tile needs, that every load stays inside x and the
router weight, and that the 8 lanes reading 8 consecutive rows of one piece
use distinct LDS banks."""
import numpy as np
import pytest

RC = 4  # k-steps per chunk


def _copies(rows_base, n_rows_valid, H, c):
    """{(copy q, slot) -> (row, element)} for one wave's 4 x-style copies of
    chunk c (two 8-row halves x two k-step pairs), rows clamped."""
    lane = np.arange(64)
    crow, cpiece = lane // 8, (lane % 8) ^ (lane // 8)
    out = {}
    for q in range(RC):
        pr, half = q % (RC // 2), q // (RC // 2)
        row = np.minimum(rows_base + 8 * half + crow, n_rows_valid - 1)
        elem = c * RC * 32 + pr * 64 + cpiece * 8
        assert (elem >= 0).all() and (elem + 8 <= H).all()
        for l in range(64):
            out[(q, l)] = (int(row[l]), int(elem[l]))
    return out


@pytest.mark.parametrize("H,T", [(2048, 64), (4096, 40), (512, 13)])
def test_router_fragments_read_what_the_tile_needs(H, T):
    lane = np.arange(64)
    nchunk = H // 32 // RC
    for c in range(nchunk):
        held = _copies(0, T, H, c)
        for s in range(RC):
            xq = ((lane % 16) // 8) * (RC // 2) + s // 2
            slot = (lane % 8) * 8 + (((s % 2) * 4 + lane // 16) ^ (lane % 8))
            for l in range(64):
                row, elem = held[(int(xq[l]), int(slot[l]))]
                assert row == min(l % 16, T - 1)
                assert elem == (c * RC + s) * 32 + (l // 16) * 8


def test_router_weight_copies_cover_each_tile_once():
    """The router weight copies of one chunk (16*ET experts, ET*RC copies of
    1 KB split over the four waves) hold every (expert, k-step, piece) of the
    chunk exactly once, rows clamped to E - 1."""
    E, H, ET = 40, 512, 4
    lane = np.arange(64)
    crow, cpiece = lane // 8, (lane % 8) ^ (lane // 8)
    w_copies = ET * RC // 4
    seen = {}
    for wave in range(4):
        for j in range(w_copies):
            f = wave * w_copies + j
            pr, half, tile = f % (RC // 2), (f // (RC // 2)) % 2, f // RC
            rows = 16 * tile + 8 * half + crow
            for l in range(64):
                key = (int(rows[l]), pr * 64 + int(cpiece[l]) * 8)
                assert key not in seen
                seen[key] = (f, l)
    assert len(seen) == 16 * ET * RC * 4  # rows x (4 pieces per k-step x RC k-steps)
    assert max(r for r, _ in seen) < 16 * ET


def test_fragment_reads_of_eight_rows_use_distinct_banks():
    lane = np.arange(64)
    for s in range(RC):
        slot = (lane % 8) * 8 + (((s % 2) * 4 + lane // 16) ^ (lane % 8))
        for g in range(0, 64, 8):
            banks = ((slot[g:g + 8] * 16) // 4) % 64 // 4  # 16-byte bank groups
            assert len(set(banks.tolist())) == 8
