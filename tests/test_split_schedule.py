"""Host-side check of the joint-attention work split (no GPU).

On the block path the attention launch may run a persistent grid of one workgroup per CU.  The
grid is cut into segments (one per XCD); each segment takes a contiguous block of (head, query
tile) units, runs whole units for its full rounds but one and splits the remaining units' key tiles
evenly over its workgroups.  A unit cut between workgroups is finished by its owner (the workgroup
holding its first key tiles), which merges the other pieces' partial online-softmax states.

This file replays that schedule in Python, with the formulas the kernel's driver uses, and checks
the properties the kernel relies on: every key tile of every unit is computed exactly once, each
workgroup publishes at most one partial and owns at most one split unit, an owner's merge loop
visits exactly the workgroups that hold its unit's other pieces, and all of them sit in the owner's
segment (so partials and flags are indexed within it).
"""
import pytest


def sk_begin(S, j, G):
    return S * j // G


def xcd_remap(bid, nwg):
    x, idx = bid & 7, bid >> 3
    q, r = nwg >> 3, nwg & 7
    return x * q + min(x, r) + idx


def plan(units, k_tiles, G):
    """The launcher's choice: (sk_grid, sk_segs); sk_grid 0 means one workgroup per unit."""
    if G <= 0 or units % G == 0:
        return 0, 1
    rounds = (units + G - 1) // G
    work = units * k_tiles
    idle = rounds * G * k_tiles - work
    if idle >= 4 * G and work >= 8 * G:
        return G, (8 if G % 8 == 0 else 1)
    return 0, 1


def schedule(units, k_tiles, G, segs):
    """Items per workgroup: (kind, unit, kb, ke, merge list) in the driver's order."""
    I = k_tiles
    Gs = G // segs
    items = {}
    for g in range(G):
        x = g // Gs
        gb, gl = x * Gs, g - x * Gs
        u0 = units * x // segs
        Us = units * (x + 1) // segs - u0
        dp = (Us // Gs - 1) * Gs if Us >= Gs else 0
        S = (Us - dp) * I
        e = sk_begin(S, gl + 1, Gs)
        it = sk_begin(S, gl, Gs)
        out = []
        w = 0
        while True:
            if gl + w * Gs < dp:
                out.append(("full", u0 + gl + w * Gs, 0, I, []))
            else:
                if it >= e:
                    break
                t = it // I
                kb = it - t * I
                ke = min(I, e - t * I)
                kind = "partial" if kb > 0 else ("full" if ke == I else "owner")
                t_end = (t + 1) * I
                merges = []
                if kind == "owner":
                    jn = gl + 1
                    while jn < Gs and sk_begin(S, jn, Gs) < t_end:
                        if sk_begin(S, jn + 1, Gs) != sk_begin(S, jn, Gs):
                            merges.append(gb + jn)
                        jn += 1
                out.append((kind, u0 + dp + t, kb, ke, merges))
                it = t * I + ke
            w += 1
        items[g] = out
    return items


CASES = [
    # (heads, query tokens, key tokens) of joint attention over text + image tokens
    ("c1 512+1024", 24, 1536, 1536),
    ("c2 512+4096", 24, 4608, 4608),
    ("c4 512+16384", 24, 16896, 16896),
    ("ragged 77+4000", 24, 4077, 4077),
    ("few heads", 3, 9000, 9000),
]


@pytest.mark.parametrize("name,heads,nq_tok,nk_tok", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("G", [256, 240, 80])
def test_attention_split_covers_every_key_tile_once(name, heads, nq_tok, nk_tok, G):
    units = heads * ((nq_tok + 255) // 256)
    k_tiles = (nk_tok + 63) // 64
    sk_grid, segs = plan(units, k_tiles, G)
    if sk_grid == 0:
        pytest.skip("the launcher keeps one workgroup per unit here")
    assert sorted(xcd_remap(b, G) for b in range(G)) == list(range(G))
    items = schedule(units, k_tiles, G, segs)
    Gs = G // segs
    cover = {}
    owner_of = {}
    pieces_of = {}
    for g, its in items.items():
        assert sum(1 for it in its if it[0] == "partial") <= 1, "one partial slot per workgroup"
        assert sum(1 for it in its if it[0] == "owner") <= 1, "one carry slot per workgroup"
        for kind, L, kb, ke, merges in its:
            assert 0 <= L < units and 0 <= kb < ke <= k_tiles
            for k in range(kb, ke):
                assert (L, k) not in cover, f"unit {L} key tile {k} computed twice"
                cover[(L, k)] = g
            if kind == "owner":
                assert L not in owner_of
                owner_of[L] = (g, merges)
            if kind == "partial":
                pieces_of.setdefault(L, []).append(g)
    assert len(cover) == units * k_tiles, "some key tile is never computed"
    for L, gs in pieces_of.items():
        g, merges = owner_of[L]
        assert merges == sorted(gs), f"unit {L}: owner {g} merges {merges}, pieces at {sorted(gs)}"
        assert all(m // Gs == g // Gs for m in merges), "a piece outside the owner's segment"
    assert set(owner_of) == set(pieces_of), "an owner with no pieces or pieces with no owner"
