"""CPU model of the FP8-column kernel's index arithmetic (expert search,
candidate experts, per-lane plans, load and store ranges), run on
well-formed and malformed token offsets: every load of codes and scales and
every store of FP8 bytes and fp32 scales must stay inside its buffer.  The
model follows the kernel's integer steps: padded starts 16 (ceil(off / 16) +
e) of clamped offsets, a 64-way search per tile, 64 candidate experts, a
binary search for the last candidate at or before each 16-position chunk.
The token-block variant (mxfp4_row_to_fp8_col_tokblk) runs the same
arithmetic with padded starts 128 (ceil(off / 128) + e) and writes one fp32
scale per (channel, 128-position slot) at H (ceil(off / 128) + e) + h
ceil(n / 128) + u / 128.  With its expert table in LDS it uses a dense
layout instead (expert e at slot pst[e], the prefix sum of ceil(n_e / 128)),
modelled by check_bounds_tokblk_dense."""
import numpy as np
import pytest

TILE = 512
CHUNKS = TILE // 16


def clampT(v, T):
    return np.minimum(np.maximum(v, 0), T)


def poff(offc, e, pad=16):
    return pad * ((offc[e] + pad - 1) // pad + e)


def find_expert(offc, E, P, pad=16):
    lo, hi = 0, E
    while hi - lo > 1:
        step = (hi - lo + 63) // 64
        e = lo + np.arange(64) * step
        ok = e < hi
        le = np.zeros(64, bool)
        le[ok] = poff(offc, e[ok], pad) <= P
        last = int(np.nonzero(le)[0].max()) if le.any() else 0
        lo += last * step
        hi = min(lo + step, hi)
    return lo


def check_bounds(off, T, H, pad=16):
    tokblk = pad == 128
    E = len(off) - 1
    offc = clampT(np.asarray(off, np.int64), T)
    ptot = pad * ((T + pad - 1) // pad + E)
    ntiles = (ptot + TILE - 1) // TILE
    HB = H // 128
    npairs = (HB + 1) // 2
    code_bytes, scale_bytes, out_bytes = T * H // 2, T * H // 32, T * H
    sc_floats = H * ((T + 127) // 128 + E) if tokblk else T * H // 128
    assert ptot < 2**31
    lane = np.arange(64)
    for tile in range(ntiles):
        P0 = tile * TILE
        eb = find_expert(offc, E, P0, pad)
        e = eb + lane
        ok = e < E
        c_off = np.where(ok, offc[np.minimum(e, E - 1)], T)
        c_n = np.where(ok, np.maximum(offc[np.minimum(e + 1, E)] - c_off, 0), 0)
        c_poff = np.where(ok, pad * ((c_off + pad - 1) // pad + e), 2**31 - 1)
        idx = np.zeros(CHUNKS, np.int64)          # binary search over the 64 candidates
        for q in range(CHUNKS):
            i, thr = 0, P0 + 16 * q
            for st in (32, 16, 8, 4, 2, 1):
                i = i + st if c_poff[i + st] <= thr else i
            idx[q] = i
        for bp in range(npairs):
            for wave in range(16):
                s8 = lane & 7
                g = 8 * wave + (lane >> 3)
                q1 = g >> 2
                i1 = idx[q1]
                off1, n1 = c_off[i1], c_n[i1]
                u1 = P0 + 16 * q1 - c_poff[i1] + 4 * (g & 3)
                b = 2 * bp + (s8 >> 2)
                for k in range(4):
                    u = u1 + k
                    val = (b < HB) & (u >= 0) & (u < n1)
                    t = off1 + u
                    a = t * (H // 2) + 128 * bp + 16 * s8
                    assert np.all(~val | ((a >= 0) & (a + 16 <= code_bytes)))
                    a = t * (H // 32) + 4 * b
                    assert np.all(~val | ((a >= 0) & (a + 4 <= scale_bytes)))
                if not tokblk:
                    u = u1 + (s8 & 3)
                    val = (b < HB) & (u >= 0) & (u < n1)
                    a = HB * off1 + b * n1 + u
                    assert np.all(~val | ((a >= 0) & (a < sc_floats)))
                if tokblk and wave == 0:
                    # scale of channel 256 bp + c for slot ts: thread (ts, c)
                    for ts in range(4):
                        i = idx[8 * ts]
                        u, n = P0 + 128 * ts - c_poff[i], c_n[i]
                        if not (0 <= u < n):
                            continue
                        h = 256 * bp + np.arange(256)
                        h = h[h < H]
                        nb = (n + 127) // 128
                        a = H * ((P0 + 128 * ts - u) // 128) + h * nb + u // 128
                        assert np.all((a >= 0) & (a < sc_floats)), (tile, ts)
                q2 = lane & 31
                i2 = idx[q2]
                off2, n2 = c_off[i2], c_n[i2]
                u2 = P0 + 16 * q2 - c_poff[i2]
                blk_ok = 2 * bp + (wave >> 3) < HB
                L = np.where(blk_ok & (u2 >= 0), np.minimum(np.maximum(n2 - u2, 0), 16), 0)
                for k in range(8):
                    h = 256 * bp + 16 * wave + 2 * k + (lane >> 5)
                    a = H * off2 + u2 + h * n2
                    assert np.all((L == 0) | ((a >= 0) & (a + L <= out_bytes)))


def find_expert_dense(pst, E, P):
    """Last expert whose dense start 128 pst[e] is at or before P (64-way)."""
    lo, hi = 0, E
    while hi - lo > 1:
        step = (hi - lo + 63) // 64
        e = lo + np.arange(64) * step
        le = (e < hi) & (128 * pst[np.minimum(e, E)] <= P)
        last = int(np.nonzero(le)[0].max()) if le.any() else 0
        lo += last * step
        hi = min(lo + step, hi)
    return lo


def check_bounds_tokblk_dense(off, T, H):
    """The token-block kernel with its expert table in LDS: expert e starts at
    slot pst[e], the exclusive prefix sum of ceil(n_e / 128) over clamped
    offsets; if that layout is longer than ceil(T / 128) + E slots (possible
    only for malformed offsets) the kernel keeps the closed form, modelled by
    check_bounds(pad=128).  Per tile the four slots' experts are searched,
    and each lane takes its slot's.  Returns whether the dense layout was
    used."""
    E = len(off) - 1
    offc = clampT(np.asarray(off, np.int64), T)
    n = np.maximum(offc[1:] - offc[:-1], 0)
    pst = np.concatenate([[0], np.cumsum((n + 127) // 128)])
    if pst[E] > (T + 127) // 128 + E:
        check_bounds(off, T, H, pad=128)
        return False
    ntiles = (int(pst[E]) + 3) // 4
    HB = H // 128
    npairs = (HB + 1) // 2
    code_bytes, scale_bytes, out_bytes = T * H // 2, T * H // 32, T * H
    sc_floats = H * ((T + 127) // 128 + E)
    lane = np.arange(64)
    for tile in range(ntiles):
        P0 = tile * TILE
        se = np.array([find_expert_dense(pst, E, P0 + 128 * k) for k in range(4)])
        assert np.all((se >= 0) & (se < E))
        s_off = offc[se]
        s_n = np.maximum(offc[se + 1] - s_off, 0)
        s_poff = 128 * pst[se]
        # each slot lies inside its expert's range or past its end (padding)
        for k in range(4):
            assert s_poff[k] <= P0 + 128 * k
            assert P0 + 128 * k + 128 <= s_poff[k] + 128 * ((s_n[k] + 127) // 128) or \
                P0 + 128 * k >= s_poff[k] + s_n[k]
        for bp in range(npairs):
            for wave in range(16):
                s8 = lane & 7
                g = 8 * wave + (lane >> 3)
                k1 = g >> 5
                off1, n1, e1 = s_off[k1], s_n[k1], se[k1]
                u1 = P0 + 4 * g - s_poff[k1]
                b = 2 * bp + (s8 >> 2)
                for k in range(4):
                    u = u1 + k
                    val = (b < HB) & (u >= 0) & (u < n1)
                    t = off1 + u
                    a = t * (H // 2) + 128 * bp + 16 * s8
                    assert np.all(~val | ((a >= 0) & (a + 16 <= code_bytes)))
                    a = t * (H // 32) + 4 * b
                    assert np.all(~val | ((a >= 0) & (a + 4 <= scale_bytes)))
                if wave % 4 == 0:
                    # thread (ts, c) with ts = wave / 4: the slot's first local
                    # index and expert come from the lane 0 plan of that wave
                    ts = wave // 4
                    u, nn = u1[0], n1[0]
                    if 0 <= u < nn:
                        h = 256 * bp + np.arange(256)
                        h = h[h < H]
                        nb = (nn + 127) // 128
                        a = H * ((off1[0] + 127) // 128 + e1[0]) + h * nb + u // 128
                        assert np.all((a >= 0) & (a < sc_floats)), (tile, ts)
                q2 = lane & 31
                k2 = q2 >> 3
                off2, n2 = s_off[k2], s_n[k2]
                u2 = P0 + 16 * q2 - s_poff[k2]
                blk_ok = 2 * bp + (wave >> 3) < HB
                L = np.where(blk_ok & (u2 >= 0), np.minimum(np.maximum(n2 - u2, 0), 16), 0)
                for k in range(8):
                    h = 256 * bp + 16 * wave + 2 * k + (lane >> 5)
                    a = H * off2 + u2 + h * n2
                    assert np.all((L == 0) | ((a >= 0) & (a + L <= out_bytes)))
    return True


MALFORMED = [
    [0, 50, 20, 90, 90],                    # a descending step
    [0, 300, 1000, 40, 600],                # beyond T, then back
    [-30, 10, 10, 600, 5000],               # negative first offset, last beyond T
    [400, 100, 0, 600],                     # off[0] != 0, descending
]


@pytest.mark.parametrize("off", MALFORMED + [[0, 3, 3, 200, 513, 600]])
@pytest.mark.parametrize("H", [128, 384])
@pytest.mark.parametrize("pad", [16, 128])
def test_accesses_stay_in_bounds(off, H, pad):
    check_bounds(np.array(off, np.int64), 600, H, pad)


def test_many_experts_and_seams():
    rng = np.random.default_rng(1)
    counts = rng.integers(0, 9, size=300)
    off = np.concatenate([[0], np.cumsum(counts)])
    for pad in (16, 128):
        check_bounds(off, int(off[-1]), 256, pad)
        off2 = off.copy()
        rng.shuffle(off2[1:-1])             # non-monotone interior
        check_bounds(off2, int(off[-1]), 256, pad)


@pytest.mark.parametrize("off", MALFORMED + [[0, 3, 3, 200, 513, 600]])
@pytest.mark.parametrize("H", [128, 384])
def test_tokblk_dense_layout_accesses_stay_in_bounds(off, H):
    check_bounds_tokblk_dense(np.array(off, np.int64), 600, H)


def test_tokblk_dense_layout_runs_of_empty_experts():
    """Long runs of experts without tokens share one start in the dense
    layout; the per-slot search still finds the expert that holds each
    slot."""
    counts = np.zeros(600, np.int64)
    counts[[5, 86, 87, 300, 598]] = [100, 60, 1, 129, 3]
    counts[400:470] = 1
    off = np.concatenate([[0], np.cumsum(counts)])
    assert check_bounds_tokblk_dense(off, int(off[-1]), 256)
    rng = np.random.default_rng(2)
    counts = rng.integers(0, 9, size=300)
    counts[rng.choice(300, 200, replace=False)] = 0
    off = np.concatenate([[0], np.cumsum(counts)])
    assert check_bounds_tokblk_dense(off, int(off[-1]), 384)
    off2 = off.copy()
    rng.shuffle(off2[1:-1])                 # non-monotone interior
    check_bounds_tokblk_dense(off2, int(off[-1]), 384)
