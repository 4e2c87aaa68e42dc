"""CPU replay of the grouped GEMM kernels' load addresses.

Every load the kernels issue must lie inside its operand, including loads
whose values are thrown away afterwards (the kernels load unconditionally
from clamped addresses and zero out-of-range values with a select). These
tests recompute, with numpy, the element offset of every 16-byte load of the
32-row kernel (grouped_gemm_kernel, the only one whose K tile of 64 can
straddle the end of a row: the down projection with I % 64 == 32), of the
skinny 16-row kernel and of the wide kernel's direct-to-LDS copies, from the
same index formulas as the HIP source, over a routing produced by the CPU
oracle's grouping, and check them against the buffer sizes the library
documents (x: T*H, act: cap*I, packed weights: E*N*K elements). The gate/up
wide kernel's act stores, taken straight from the accumulators, are replayed
the same way."""
import numpy as np
import pytest

import oracle


def _routing(T, k, E, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    sorted_ids, block_expert, _, npad = oracle.align(ids, E, bm)
    return sorted_ids, block_expert, npad


def _frag_index(r, c, cols):
    r = np.asarray(r, np.int64)
    c = np.asarray(c, np.int64)
    return ((r >> 4) * (cols >> 5) + (c >> 5)) * 512 + ((((c & 31) >> 3) << 4) + (r & 15)) * 8 + (c & 7)


def _check(offsets, numel, what):
    offsets = np.asarray(offsets, np.int64)
    assert offsets.min() >= 0, f"{what}: load before the buffer ({offsets.min()})"
    assert offsets.max() + 8 <= numel, f"{what}: load ends at element {offsets.max() + 8}, buffer has {numel}"


def _general_kernel_loads(gated, sorted_ids, block_expert, npad, T, k, K, N_out, E):
    """All A and B load offsets of grouped_gemm_kernel<GemmCfg<32, 128, gated>>."""
    BM, BN, BK, THREADS, KS = 32, 128, 64, 256, 2
    n_tiles = -(-N_out // (BN // 2 if gated else BN))
    w_rows = 2 * N_out if gated else N_out
    bands = w_rows // 16
    n_pairs = T * k
    nk = -(-K // BK)
    tid = np.arange(THREADS)
    a_offs, b_offs = [], []
    for mb in range(len(block_expert)):
        if mb * BM >= npad or block_expert[mb] < 0:
            continue
        e = int(block_expert[mb])
        ids = sorted_ids[mb * BM:(mb + 1) * BM]
        real = (ids >= 0) & (ids < n_pairs)
        row_src = np.where(real, (ids // k) * K, -1) if gated else np.where(real, ids, -1)
        # A: one chunk per thread (A_CHUNKS = 256)
        row, kc = tid // (BK // 8), (tid % (BK // 8)) * 8
        if gated:
            src = row_src[row]
            a_ptr = np.where(src >= 0, src, 0) + kc
        else:
            a_ptr = _frag_index(mb * BM + row, kc, K)
        for kt in range(nk):
            k0 = kt * BK
            inr = k0 + kc < K
            off = np.where(inr, k0, 0) if gated else np.where(inr, k0 * 16, -(kc >> 5) * 512)
            a_offs.append(a_ptr + off)
        for tn in range(n_tiles):
            for j in range(4):  # B_PER_T
                c = np.minimum(tid + j * THREADS, BN * BK // 8 - 1)
                band = np.minimum(tn * (BN // 16) + c // (KS * 64), bands - 1)
                b_ptr = e * w_rows * K + band * 16 * K + ((c // 64) % KS) * 512 + (c % 64) * 8
                ks = ((tid + j * THREADS) // 64) % KS
                for kt in range(nk):
                    inr = kt * KS + ks < K // 32
                    b_offs.append(b_ptr + np.where(inr, kt * KS * 512, -ks * 512))
    return np.concatenate(a_offs), np.concatenate(b_offs)


@pytest.mark.parametrize("T,H,E,k,I", [(20, 64, 8, 8, 32), (37, 128, 8, 2, 96), (64, 256, 16, 4, 160),
                                       (300, 192, 12, 3, 224)])
def test_general_kernel_down_loads_in_bounds(T, H, E, k, I):
    """Down projection through the 32-row kernel with I % 64 == 32: the last
    K tile's second half lies past each act row and each weight band."""
    bm = 32
    sorted_ids, block_expert, npad = _routing(T, k, E, bm, T + I)
    cap = len(sorted_ids)
    # worst case for the act operand: padded rows fill the whole capacity
    a, b = _general_kernel_loads(False, sorted_ids, block_expert, npad, T, k, I, H, E)
    _check(a, cap * I, "act")
    _check(b, E * H * I, "w2")


@pytest.mark.parametrize("T,H,E,k,I", [(20, 64, 8, 8, 32), (64, 256, 16, 4, 160)])
def test_general_kernel_gate_up_loads_in_bounds(T, H, E, k, I):
    bm = 32
    sorted_ids, block_expert, npad = _routing(T, k, E, bm, T + H)
    a, b = _general_kernel_loads(True, sorted_ids, block_expert, npad, T, k, H, I, E)
    _check(a, T * H, "x")
    _check(b, E * 2 * I * H, "w13")


def test_general_kernel_down_tail_when_capacity_is_full():
    """Every expert gets exactly a multiple of 32 rows, so num_padded equals
    the capacity's real part and the last row band ends the act buffer."""
    T, H, E, k, I = 32, 64, 8, 8, 32
    ids = np.tile(np.arange(8, dtype=np.int32), (T, 1))
    sorted_ids, block_expert, _, npad = oracle.align(ids, E, 32)
    a, b = _general_kernel_loads(False, sorted_ids, block_expert, npad, T, k, I, H, E)
    _check(a, npad * I, "act (exactly num_padded rows)")
    _check(b, E * H * I, "w2")


def _skinny_loads(gated, sorted_ids, block_expert, npad, T, k, K, N_out, E, NW, NTILE):
    lane = np.arange(64)
    w_rows = 2 * N_out if gated else N_out
    bands = w_rows // 16
    cols = 8 * NTILE if gated else 16 * NTILE
    n_tiles = -(-N_out // (NW * cols))
    n_pairs = T * k
    a_offs, b_offs = [], []
    for mb in range(len(block_expert)):
        if mb * 16 >= npad or block_expert[mb] < 0:
            continue
        e = int(block_expert[mb])
        ids = sorted_ids[mb * 16 + lane % 16]
        ok = (ids >= 0) & (ids < n_pairs)
        if gated:
            ap = np.where(ok, (ids // k) * K, 0) + (lane // 16) * 8
            step = 32
        else:
            ap = mb * (K // 32) * 512 + lane * 8
            step = 512
        for s in range(K // 32):
            a_offs.append(ap + s * step)
        for tn in range(n_tiles):
            for wave in range(NW):
                c0 = (tn * NW + wave) * cols
                for j in range(NTILE):
                    band = 2 * (c0 // 16 + j % (NTILE // 2)) + (0 if j < NTILE // 2 else 1) if gated else c0 // 16 + j
                    bp = e * w_rows * K + min(band, bands - 1) * 16 * K + lane * 8
                    for s in range(K // 32):
                        b_offs.append(bp + s * 512)
    return np.concatenate(a_offs), np.concatenate(b_offs)


@pytest.mark.parametrize("T,H,E,k,I", [(20, 64, 8, 8, 32), (45, 128, 1, 1, 64), (33, 1024, 256, 32, 32)])
def test_skinny_kernel_loads_in_bounds(T, H, E, k, I):
    sorted_ids, block_expert, npad = _routing(T, k, E, 16, T)
    cap = len(sorted_ids)
    a, b = _skinny_loads(True, sorted_ids, block_expert, npad, T, k, H, I, E, 1, 2)
    _check(a, T * H, "x")
    _check(b, E * 2 * I * H, "w13")
    a, b = _skinny_loads(False, sorted_ids, block_expert, npad, T, k, I, H, E, 4, 4)
    _check(a, cap * I, "act")
    _check(b, E * H * I, "w2")


def _wide_copies(gated, bm, sorted_ids, block_expert, npad, T, k, K, N_out, E, bn=512, am=1):
    """Byte offsets of the wide kernel's direct-to-LDS copies (activations
    relative to x or act, weights relative to the whole packed weight). bm
    is the tile's rows; with am = 2 the grouping blocks are 2*bm rows (block_m
    256 computed as two 128-row tiles) and block_expert is indexed per
    grouping block."""
    lane = np.arange(64)
    w_rows = 2 * N_out if gated else N_out
    bands = w_rows // 16
    cols = bn // 2 if gated else bn
    n_tiles = -(-N_out // cols)
    n_pairs = T * k
    a_offs, b_offs = [], []
    for mb in range(npad // bm):
        e = int(block_expert[mb // am])
        assert e >= 0
        for tn in range(n_tiles):
            band0 = tn * (bn // 16)
            for q in range((bm + bn) // 16):
                if q < bm // 16:
                    if gated:
                        row = q * 16 + lane // 4
                        chunk = (lane % 4) ^ ((row >> 2) & 3)
                        ids = sorted_ids[mb * bm + row]
                        real = (ids >= 0) & (ids < n_pairs)
                        soff = (np.where(real, (ids // k) * K, 0) + chunk * 8) * 2
                        step = 64
                    else:
                        soff = ((mb * (bm // 16) + q) * (K // 32) * 512 + lane * 8) * 2
                        step = 1024
                    for kt in range(K // 32):
                        a_offs.append(soff + kt * step)
                else:
                    band = min(band0 + q - bm // 16, bands - 1)
                    soff = e * w_rows * K * 2 + (band * 16 * K + lane * 8) * 2
                    for kt in range(K // 32):
                        b_offs.append(soff + kt * 1024)
    return np.concatenate(a_offs) // 2, np.concatenate(b_offs) // 2


@pytest.mark.parametrize("bm", [64, 128])
@pytest.mark.parametrize("T,H,E,k,I", [(700, 192, 8, 2, 160), (520, 128, 4, 1, 96)])
def test_wide_kernel_copies_in_bounds(bm, T, H, E, k, I):
    sorted_ids, block_expert, npad = _routing(T, k, E, bm, T + bm)
    cap = len(sorted_ids)
    bn = 256 if bm == 64 else 512  # weight rows per tile: 64x256 and 128x512 tiles
    a, b = _wide_copies(True, bm, sorted_ids, block_expert, npad, T, k, H, I, E, bn=bn)
    _check(a, T * H, "x")
    _check(b, E * 2 * I * H, "w13")
    a, b = _wide_copies(False, bm, sorted_ids, block_expert, npad, T, k, I, H, E, bn=bn)
    _check(a, cap * I, "act")
    _check(b, E * H * I, "w2")
    # quarter-width down tiles: 128 weight rows from band tn*32 + sub*8
    a, b = _wide_copies(False, bm, sorted_ids, block_expert, npad, T, k, I, H, E, bn=128)
    _check(b, E * H * I, "w2 (quarter tiles)")


def test_wide_kernel_copies_in_bounds_block_m_256():
    T, H, E, k, I = 700, 192, 8, 2, 160
    sorted_ids, block_expert, npad = _routing(T, k, E, 256, T)
    cap = len(sorted_ids)
    a, b = _wide_copies(True, 128, sorted_ids, block_expert, npad, T, k, H, I, E, am=2)
    _check(a, T * H, "x")
    _check(b, E * 2 * I * H, "w13")
    a, b = _wide_copies(False, 128, sorted_ids, block_expert, npad, T, k, I, H, E, am=2)
    _check(a, cap * I, "act")
    _check(b, E * H * I, "w2")



def _wide_act_stores(bm, tm, waves_n, wtn, npad, N_out, col_tiles):
    """Element offsets of act written by the gate/up wide kernel's epilogue
    (straight from the accumulators: lane l holds row l%32 of each 32-row
    block and four consecutive columns 8*c8 + 4*(l/32) .. +3 of each
    32-column block), with the logical (row, column) of each."""
    lane = np.arange(64)
    waves_m = bm // (32 * tm)
    offs, rows, cols = [], [], []
    for mb in range(npad // bm):
        for col0 in col_tiles:
            for wm in range(waves_m):
                for wn in range(waves_n):
                    for i in range(tm):
                        R = mb * bm + wm * 32 * tm + i * 32 + lane % 32
                        for g in range(wtn // 64):
                            cb = col0 + wn * (wtn // 2) + g * 32
                            if cb >= N_out:
                                continue
                            for c8 in range(4):
                                for u in range(4):
                                    offs.append(((R // 16) * (N_out // 32) + cb // 32) * 512 + (R % 16) * 8 +
                                                4 * (lane // 32) + c8 * 128 + u)
                                    rows.append(R)
                                    cols.append(cb + 8 * c8 + 4 * (lane // 32) + u)
    return np.concatenate(offs), np.concatenate(rows), np.concatenate(cols)


@pytest.mark.parametrize("bm", [64, 128])
@pytest.mark.parametrize("T,H,E,k,I", [(700, 192, 8, 2, 160), (520, 128, 4, 1, 96), (300, 256, 16, 4, 288)])
def test_wide_kernel_act_stores_cover_rows_once(bm, T, H, E, k, I):
    """The act stores of gate/up write every element of rows [0, num_padded)
    exactly once (pad rows as zeros), each at its fragment-layout offset."""
    _, _, npad = _routing(T, k, E, bm, T + bm + I)
    if bm == 128:  # 8 waves as 2 x 4 with 64x128 wave tiles, 256 output columns per tile
        offs, rows, cols = _wide_act_stores(bm, 2, 4, 128, npad, I, range(0, I, 256))
    else:  # 64x256 tiles: 4 waves as 2 x 2 with 32x128 wave tiles, 128 output columns
        offs, rows, cols = _wide_act_stores(bm, 1, 2, 128, npad, I, range(0, I, 128))
    assert np.array_equal(offs, _frag_index(rows, cols, I)), "act offsets follow the fragment layout"
    assert np.array_equal(np.sort(offs), np.arange(npad * I)), "every act element of the real blocks once"
