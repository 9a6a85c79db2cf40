"""Host-side model of the head-major attention kernel's tile loads (the per-lane source offsets of
sparse_attn_kernel's global->LDS loads, written out here in NumPy), checked against the sizes of
the buffers they read: every load of the kernel's own tile schedule stays inside q/kv/k_pe/bitmap;
the persistent schedule covers every query tile once, and the key-tile lists built from the flags
stay below each item's tile count. No GPU is used.

The last check names the mechanism behind an access fault seen once with an experimental L2
prefetch of tile t+4 (the variant is not in the library), on the load form the kernel had then:
offsets relative to the tile's first row, rows clamped by min(row, T - 1 - t0). At T = 200 such a
tile starts at key 256, past the last key 199, so that clamp is negative for every row; the 32-bit
per-lane offset of the scalar-base load then wraps around (the hardware adds it zero-extended), and
the selection words of tile t+4 lie past the bitmap of the last sequence. The kernel now takes
offsets from the head's first row and clamps the absolute row, min(t0 + row, T - 1), so key and
rotary rows of any tile index stay inside their buffers; its schedule only ever loads tiles below
the item's tile count, which keeps the bitmap words in bounds as well."""
import numpy as np
import pytest

KT, QT, WAVES, ROPE = 64, 256, 8, 64
KV_ROW = 512          # bytes per key row of one head: 128 key + 128 value bf16
KP_ROW = 2 * ROPE


def bitmap_geometry(T):
    return 2 * ((T + KT - 1) // KT), (T + QT - 1) // QT * QT     # words per column, columns


def tile_loads(B, T, b, h, kt, q0):
    """Byte offsets (relative to each buffer's start) of every 16-byte load one workgroup issues
    for key tile kt of item (b, h, query tile starting at q0): [(buffer, offsets), ...]. Scalar
    bases: the head's first key row, the sequence's first rotary row, the item's first bitmap
    column; per-lane 32-bit offsets from there."""
    lane = np.arange(64)
    r16 = lane >> 4
    t0 = kt * KT
    Wp, Tpad = bitmap_geometry(T)
    out = []
    for wave in range(WAVES):
        kn_wave = wave < 4
        for k in range(4):
            row = 16 * (wave & 3) + 4 * k + r16
            lc = (lane & 15) ^ ((4 * k + r16) & 15) if kn_wave else (lane & 15) ^ (4 * r16)
            chunk = lc * 16 + (0 if kn_wave else 256)
            voff = (np.minimum(t0 + row, T - 1).astype(np.uint64) * 512 + chunk.astype(np.uint64)) & 0xFFFFFFFF
            out.append(("kv", (b * 128 + h) * T * 256 * 2 + voff))
        kp_row = 8 * wave + (lane >> 3)
        kp_chunk = ((lane & 7) ^ ((kp_row >> 1) & 7)) << 4
        voff = (np.minimum(t0 + kp_row, T - 1).astype(np.uint64) * KP_ROW + kp_chunk.astype(np.uint64)) & 0xFFFFFFFF
        out.append(("k_pe", b * T * ROPE * 2 + voff))
        if wave < 2:
            voff = (np.uint64((kt * 2 + wave) * Tpad * 4) + lane.astype(np.uint64) * 16) & 0xFFFFFFFF
            out.append(("bitmap", (b * Wp * Tpad + q0) * 4 + voff))
    return out


def tile_loads_relative_rows(B, T, b, h, kt, q0):
    """The same loads in the form the kernel had when the prefetch variant faulted: scalar bases
    at the tile's first row, per-lane offsets relative to it with rows clamped by
    min(row, T - 1 - t0)."""
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


def units_of_workgroups(B, T, G):
    """The kernel's persistent schedule: for workgroup w, its units u = w, w + G, ... as
    (b, h, pair) in the order it runs them."""
    nqt = (T + QT - 1) // QT
    npairs = (nqt + 1) // 2
    BH = B * 128
    units = 8 * ((BH + 7) // 8) * npairs
    per_wg = []
    for w in range(G):
        mine = []
        for u in range(w, units, G):
            k = u >> 3
            grp = k // npairs
            bh = (u & 7) + 8 * grp
            j0 = ((u & 7) + 8 * grp * npairs) // G
            pr = (k - grp * npairs + j0) % npairs
            if bh < BH:
                mine.append((bh // 128, bh % 128, pr))
        per_wg.append(mine)
    return per_wg, nqt, npairs


@pytest.mark.parametrize("B,T,G", [(2, 4096, 256), (1, 1100, 256), (1, 16384, 256), (3, 130, 256),
                                   (2, 2400, 256), (1, 32768, 256), (2, 4096, 248), (1, 5000, 80)])
def test_persistent_schedule_covers_every_query_tile_once(B, T, G):
    """Every (b, h, query tile) is computed by exactly one workgroup: a unit is query tile
    nqt-1-p then p (once when they coincide), and the pair rotation is a permutation per head."""
    per_wg, nqt, npairs = units_of_workgroups(B, T, G)
    seen = {}
    for w, mine in enumerate(per_wg):
        for b, h, pr in mine:
            tiles = [nqt - 1 - pr] + ([pr] if pr != nqt - 1 - pr else [])
            for qt in tiles:
                assert (b, h, qt) not in seen, (b, h, qt, w, seen.get((b, h, qt)))
                seen[(b, h, qt)] = w
    assert len(seen) == B * 128 * nqt


def test_persistent_schedule_gives_each_workgroup_every_pair_at_the_headline():
    """At B=2, T=4096 on 256 workgroups (8 pairs, 32 workgroups per XCD) each workgroup runs each
    pair once, so pair costs that differ (skipped key tiles) even out; and at every step the
    workgroups of one XCD share 4 heads, all 8 pairs of each."""
    per_wg, nqt, npairs = units_of_workgroups(2, 4096, 256)
    assert npairs == 8
    for mine in per_wg:
        assert sorted(pr for _, _, pr in mine) == list(range(8))
    for x in range(8):
        for j in range(8):
            step = [per_wg[w][j] for w in range(x, 256, 8)]
            heads = {(b, h) for b, h, _ in step}
            assert len(heads) == 4 and all(h % 8 == x for _, h in heads)
            for bh in heads:
                assert sorted(pr for b, h, pr in step if (b, h) == bh) == list(range(8))


def key_tile_list(flag_words, nkt):
    """The list the kernel's wave 0 builds from an item's flag words: tiles below nkt whose bit is
    set, ascending; {0} when none is."""
    lst = [kt for kt in range(nkt) if (int(flag_words[kt // 32]) >> (kt % 32)) & 1]
    return lst or [0]


def test_key_tile_lists_stay_below_the_item_tile_count():
    """Whatever the flags hold (even bits past the causal limit, which the selection kernels never
    set), the tiles an item loads are among 0..nkt-1, whose loads the schedule test above checks,
    and the flag words read are inside the item's row of ceil(ceil(T/64) / 32) words."""
    rng = np.random.default_rng(9)
    for T in (1, 64, 200, 1100, 4096, 32768):
        nkt_total = (T + KT - 1) // KT
        fw = (nkt_total + 31) // 32
        for q0, nkt in schedule(T):
            lanes = [l for l in range(64) if 8 * l < nkt]
            assert max(l >> 2 for l in lanes) < fw
            for words in (rng.integers(0, 2 ** 32, fw, dtype=np.uint64), np.zeros(fw, np.uint64),
                          np.full(fw, 2 ** 32 - 1, np.uint64)):
                lst = key_tile_list(words, nkt)
                assert lst == sorted(set(lst)) and 0 <= lst[0] and lst[-1] < nkt


def test_a_tile_past_the_sequence_would_load_out_of_bounds():
    B, T = 2, 200
    lim = sizes(B, T)
    (q0, nkt), = schedule(T)
    assert nkt == 4
    kt = 4                                  # tile t + 4 seen from t = 0: keys 256..319 > 199
    loads = dict()
    for buf, off in tile_loads_relative_rows(B, T, B - 1, 127, kt, q0):
        loads.setdefault(buf, []).append(off)
    kv = np.concatenate(loads["kv"])
    kp = np.concatenate(loads["k_pe"])
    bm = np.concatenate(loads["bitmap"])
    # the negative row clamp wraps the 32-bit offset: about 4 GB past the tile's base
    assert kv.max() > 2 ** 31 and kv.max() + 16 > lim["kv"]
    assert kp.max() + 16 > lim["k_pe"]
    # words 8 and 9 of a bitmap with 8 words per column: past the last sequence's bitmap
    assert bm.max() + 16 > lim["bitmap"]
    # the kernel's present form clamps the absolute row: key and rotary rows stay in bounds for
    # any tile index; the bitmap words of a tile past the sequence would still not
    now = dict()
    for buf, off in tile_loads(B, T, B - 1, 127, kt, q0):
        now.setdefault(buf, []).append(off)
    assert max(o.max() for o in now["kv"]) + 16 <= lim["kv"]
    assert max(o.max() for o in now["k_pe"]) + 16 <= lim["k_pe"]
    assert max(o.max() for o in now["bitmap"]) + 16 > lim["bitmap"]


def test_both_load_forms_agree_inside_the_sequence():
    """For every tile the schedule loads, the present offsets address the same bytes as the
    earlier relative form."""
    for B, T in ((2, 200), (1, 1100), (3, 130)):
        for q0, nkt in schedule(T):
            for kt in range(nkt):
                for b, h in ((0, 0), (B - 1, 127)):
                    a = tile_loads(B, T, b, h, kt, q0)
                    r = tile_loads_relative_rows(B, T, b, h, kt, q0)
                    for (ba, oa), (br, orr) in zip(a, r):
                        assert ba == br and np.array_equal(oa, orr), (B, T, kt, ba)
