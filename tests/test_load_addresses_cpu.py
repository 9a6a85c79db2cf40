"""Host-side model of the head-major attention kernel's tile loads (the per-lane source offsets of
sparse_attn_kernel's global->LDS loads, written out here in NumPy), checked against the sizes of
the buffers they read: every load of the kernel's own tile schedule stays inside q/kv/k_pe/bitmap,
and a load of a tile that starts past the sequence would not. No GPU is used.

The second check names the mechanism behind an access fault seen once with an experimental L2
prefetch of tile t+4 (the variant is not in the library): at T = 200 such a tile starts at key 256,
past the last key 199, so the row clamp min(row, T - 1 - t0) is negative for every row; the 32-bit
per-lane offset of the scalar-base load then wraps around (the hardware adds it zero-extended), and
the selection words of tile t+4 lie past the bitmap of the last sequence."""
import numpy as np
import pytest

KT, QT, WAVES, ROPE = 64, 256, 8, 64
KV_ROW = 512          # bytes per key row of one head: 128 key + 128 value bf16
KP_ROW = 2 * ROPE


def bitmap_geometry(T):
    return 2 * ((T + KT - 1) // KT), (T + QT - 1) // QT * QT     # words per column, columns


def tile_loads(B, T, b, h, kt, q0):
    """Byte offsets (relative to each buffer's start) of every 16-byte load one workgroup issues
    for key tile kt of item (b, h, query tile starting at q0): [(buffer, offsets), ...]."""
    lane = np.arange(64)
    r16 = lane >> 4
    t0 = kt * KT
    tl = T - 1 - t0
    out = []
    for wave in range(WAVES):
        kn_wave = wave < 4
        for k in range(4):
            row = 16 * (wave & 3) + 4 * k + r16
            lc = (lane & 15) ^ ((4 * k + r16) & 15) if kn_wave else (lane & 15) ^ (4 * r16)
            src = (row * 512 + lc * 16 + (0 if kn_wave else 256)).astype(np.uint64)
            dr = np.minimum(row, tl) - row
            voff = (src + (dr * 512).astype(np.int64).astype(np.uint64)) & 0xFFFFFFFF   # 32-bit add
            base = ((b * 128 + h) * T * 256 + t0 * 256) * 2
            out.append(("kv", base + voff))
        kp_row = 8 * wave + (lane >> 3)
        kp_off = (kp_row * KP_ROW + (((lane & 7) ^ ((kp_row >> 1) & 7)) << 4)).astype(np.uint64)
        drp = np.minimum(kp_row, tl) - kp_row
        voff = (kp_off + (drp * KP_ROW).astype(np.int64).astype(np.uint64)) & 0xFFFFFFFF
        out.append(("k_pe", (b * T * ROPE + t0 * ROPE) * 2 + voff))
        if wave < 2:
            Wp, Tpad = bitmap_geometry(T)
            out.append(("bitmap", ((b * Wp + kt * 2 + wave) * Tpad + q0) * 4 + lane.astype(np.uint64) * 16))
    return out


def sizes(B, T):
    Wp, Tpad = bitmap_geometry(T)
    return {"kv": B * 128 * T * 256 * 2, "k_pe": B * T * ROPE * 2, "bitmap": B * Wp * Tpad * 4}


def schedule(T):
    """(q0, number of key tiles) of every query tile, as the kernel walks them: tiles 0 and 1,
    then tile kt + 2 while tile kt is computed, for kt + 2 below the item's tile count."""
    items = []
    for qt in range((T + QT - 1) // QT):
        q0 = qt * QT
        nkt = (min(T, q0 + QT) - 1) // KT + 1
        items.append((q0, nkt))
    return items


@pytest.mark.parametrize("B,T", [(2, 200), (1, 1), (1, 64), (3, 130), (1, 1100), (2, 4096), (1, 333)])
def test_kernel_schedule_loads_stay_in_bounds(B, T):
    lim = sizes(B, T)
    for q0, nkt in schedule(T):
        issued = [0, 1][:nkt] + [kt + 2 for kt in range(nkt) if kt + 2 < nkt]
        assert sorted(issued) == list(range(nkt))
        for b in (0, B - 1):
            for h in (0, 127):
                for kt in issued:
                    for buf, off in tile_loads(B, T, b, h, kt, q0):
                        assert off.min() >= 0 and off.max() + 16 <= lim[buf], (buf, b, h, kt, q0)


def test_a_tile_past_the_sequence_would_load_out_of_bounds():
    B, T = 2, 200
    lim = sizes(B, T)
    (q0, nkt), = schedule(T)
    assert nkt == 4
    kt = 4                                  # tile t + 4 seen from t = 0: keys 256..319 > 199
    loads = dict()
    for buf, off in tile_loads(B, T, B - 1, 127, kt, q0):
        loads.setdefault(buf, []).append(off)
    kv = np.concatenate(loads["kv"])
    kp = np.concatenate(loads["k_pe"])
    bm = np.concatenate(loads["bitmap"])
    # the negative row clamp wraps the 32-bit offset: about 4 GB past the tile's base
    assert kv.max() > 2 ** 31 and kv.max() + 16 > lim["kv"]
    assert kp.max() + 16 > lim["k_pe"]
    # words 8 and 9 of a bitmap with 8 words per column: past the last sequence's bitmap
    assert bm.max() + 16 > lim["bitmap"]
