"""Reference tile scheduler in plain Python integers.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the host load balancer of "Jagged Flash Attention for GEM" (section on
GEM-specific optimisations): every tile is given its KV work, the tiles are sorted
by that work in descending order, and they are dealt over the compute units in a
zigzag: pass 0 fills slots left to right, pass 1 right to left, and so on.

Readings of what the page leaves open:
  * A tile is one block of query rows of one (sequence, head) for the forward,
    one block of key rows for the backward.
  * Work of a forward tile = number of keys it visits: L, or with causal
    min(L, (t+1)*BM). Broadcast-Q forward tiles visit the L_b keys of their
    sequence.
  * Work of a backward tile = number of query rows that attend its keys: L, or
    with causal L - n*BN. Broadcast-Q backward tiles see all Lq query rows.
  * Ties keep generation order (sequence, then head, then tile); the sort is stable.
  * Passes are counted from 0; pass 0 runs from slot 0 upward.
  * "In-order" dispatch deals tiles in generation order round-robin: tile j goes
    to slot j mod S.
  * The XCD variant (an MI355X refinement: eight dies with separate L2s) first
    deals whole (sequence, head) units, weighted by their total work, zigzag over
    the dies, then applies the same rule inside each die's slots.
  * The folded variant (an MI355X refinement for causal problems) applies the
    same rule to items instead of tiles: with causal masking, tiles a and n-1-a
    of one (sequence, head) form one item whose work is their sum (the middle
    tile of an odd count stands alone); an item's tiles go to one slot, in that
    order. Without causal masking every tile is an item.
  * Block-sparse attention (64-token blocks, one block mask per sequence): a
    tile covers two blocks (128 query rows, or 128 keys); its step list names the
    other side's blocks that pair with either of them, ascending. A key tile's
    work is 64 times its list's length (the query rows it visits); a query tile's
    two blocks walk their own entries side by side, so its work is 64 times the
    longer of the two (the entries carrying bit 28, or bit 29).
  * The balanced in-order variant (an MI355X refinement for tiles whose cost
    depends on L2 sharing within a (sequence, head)): (sequence, head) units in
    generation order, each to the group of slots (one per XCD) with the least
    work dealt so far, the lower group on ties; the unit's tiles, in order, each
    to the least-loaded slot of that group, the lower slot on ties. With a slot
    count that is not a multiple of 8 all slots form one group.
Output: slot_ptr [S+1] and tiles [N,4] = (b, h, t, work), grouped by slot, in the
order each slot received them.
"""
from __future__ import annotations

import numpy as np

KIND_FWD, KIND_BWD = 0, 1
SPARSE_BLOCK, SPARSE_BIT = 64, 28
ORDER_INORDER, ORDER_ZIGZAG, ORDER_XCD_ZIGZAG, ORDER_FOLDED_ZIGZAG, ORDER_XCD_INORDER = 0, 1, 2, 3, 4


def ceil_div(a, b):
    return -(-a // b)


def sparse_lists(lengths, masks, kind, tile_rows=128, causal=False):
    """Block-sparse step lists: (seq_base, list_ptr, entries) as int32 arrays.

    One list per (sequence b, tile t), in that order; tile t covers the blocks
    2t and 2t+1 (query blocks for KIND_FWD, key blocks for KIND_BWD). Its entries
    are the other side's blocks c, ascending, that pair with either: the block
    index plus bit 28 when block 2t pairs with c (FWD: masks[b][2t, c]; BWD:
    masks[b][c, 2t]) and bit 29 for block 2t+1. With causal a key block never
    pairs with an earlier query block. seq_base[b] is the first list of sequence b.
    """
    seq_base, list_ptr, entries = [], [0], []
    for L, m in zip((int(x) for x in lengths), masks):
        seq_base.append(len(list_ptr) - 1)
        n = m.shape[0]
        for t in range(ceil_div(L, tile_rows)):
            for c in range(n):
                code = c
                for i, blk in enumerate((2 * t, 2 * t + 1)):
                    qb, kb = (blk, c) if kind == KIND_FWD else (c, blk)
                    if blk < n and m[qb, kb] and not (causal and kb > qb):
                        code |= 1 << (SPARSE_BIT + i)
                if code != c:
                    entries.append(code)
            list_ptr.append(len(entries))
    seq_base.append(len(list_ptr) - 1)
    return (np.asarray(seq_base, dtype=np.int32), np.asarray(list_ptr, dtype=np.int32),
            np.asarray(entries, dtype=np.int64).astype(np.int32))


def enumerate_tiles(lengths, num_heads, kind, tile_rows, causal=False, lq=0, window=0,
                    sparse_list_ptr=None, sparse_entries=None):
    """All tiles in generation order: list of (b, h, t, work).

    With a causal window W the work counts only what the window leaves: a query
    tile visits the keys from max(0, t*BM - W + 1) to its last row, a key tile is
    attended by the queries from n*BN to min(L, (n+1)*BN - 1 + W). With block-sparse
    step lists (list_ptr and entries of sparse_lists) a key tile's work is 64 times
    its list's length and a query tile's 64 times the number of its entries that
    carry bit 28 or bit 29, whichever is larger.
    """
    out = []
    if sparse_list_ptr is not None:
        u = 0
        for b, L in enumerate(int(x) for x in lengths):
            n = ceil_div(L, tile_rows)
            for h in range(num_heads):
                for t in range(n):
                    lo, hi = int(sparse_list_ptr[u + t]), int(sparse_list_ptr[u + t + 1])
                    if kind == KIND_FWD:
                        e = [int(x) for x in sparse_entries[lo:hi]]
                        steps = max(sum((x >> SPARSE_BIT) & 1 for x in e),
                                    sum((x >> (SPARSE_BIT + 1)) & 1 for x in e))
                    else:
                        steps = hi - lo
                    out.append((b, h, t, SPARSE_BLOCK * steps))
            u += n
        return out
    for b, L in enumerate(int(x) for x in lengths):
        for h in range(num_heads):
            if kind == KIND_FWD:
                if lq:
                    for t in range(ceil_div(lq, tile_rows)):
                        out.append((b, h, t, L))
                else:
                    for t in range(ceil_div(L, tile_rows)):
                        work = min(L, (t + 1) * tile_rows) if causal else L
                        if causal and window:
                            work -= max(0, t * tile_rows - window + 1)
                        out.append((b, h, t, work))
            else:
                for n in range(ceil_div(L, tile_rows)):
                    if lq:
                        work = lq
                    elif causal and window:
                        work = min(L, (n + 1) * tile_rows - 1 + window) - n * tile_rows
                    else:
                        work = L - n * tile_rows if causal else L
                    out.append((b, h, n, work))
    return out


def _zigzag_rank(j, n):
    """Position j of a zigzag deal over n places: pass j // n, rank j % n."""
    p, r = divmod(j, n)
    return n - 1 - r if p % 2 else r


def schedule(lengths, num_heads, kind, tile_rows, order, num_slots, causal=False, lq=0,
             groups=8, window=0, sparse_list_ptr=None, sparse_entries=None):
    tiles = enumerate_tiles(lengths, num_heads, kind, tile_rows, causal, lq, window,
                            sparse_list_ptr, sparse_entries)
    if order == ORDER_XCD_INORDER:
        # (sequence, head) units in generation order: each to the least-loaded
        # group, its tiles in order each to the least-loaded slot of the group
        ng = groups if num_slots % groups == 0 else 1
        per = num_slots // ng
        group_load = [0] * ng
        slot_load = [0] * num_slots
        per_slot = [[] for _ in range(num_slots)]
        g = 0
        while g < len(tiles):
            e = g
            while e < len(tiles) and tiles[e][:2] == tiles[g][:2]:
                e += 1
            x = min(range(ng), key=lambda i: (group_load[i], i))
            group_load[x] += sum(t[3] for t in tiles[g:e])
            for t in tiles[g:e]:
                s = min(range(x * per, (x + 1) * per), key=lambda i: (slot_load[i], i))
                slot_load[s] += t[3]
                per_slot[s].append(t)
            g = e
        slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
        flat = []
        for s in range(num_slots):
            flat.extend(per_slot[s])
            slot_ptr[s + 1] = len(flat)
        return slot_ptr, np.asarray(flat, dtype=np.int32).reshape(-1, 4)
    if order == ORDER_XCD_ZIGZAG:
        # Units are (sequence, head) pairs with the summed work of their tiles;
        # they are sorted by that work and dealt zigzag over the groups, then each
        # group's tiles are sorted and dealt zigzag over the group's own slots.
        assert num_slots % groups == 0
        per = num_slots // groups
        units = {}
        for g, t in enumerate(tiles):
            units.setdefault((t[0], t[1]), []).append(g)
        keys = list(units)                      # insertion order = generation order
        work = {u: sum(tiles[g][3] for g in units[u]) for u in keys}
        ranked = sorted(range(len(keys)), key=lambda i: (-work[keys[i]], i))
        group_of = {}
        for j, i in enumerate(ranked):
            group_of[keys[i]] = _zigzag_rank(j, groups)
        per_slot = [[] for _ in range(num_slots)]
        for x in range(groups):
            mine = [g for u in keys if group_of[u] == x for g in units[u]]
            mine.sort(key=lambda g: (-tiles[g][3], g))
            for j, g in enumerate(mine):
                per_slot[x * per + _zigzag_rank(j, per)].append(tiles[g])
        slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
        flat = []
        for s in range(num_slots):
            flat.extend(per_slot[s])
            slot_ptr[s + 1] = len(flat)
        return slot_ptr, np.asarray(flat, dtype=np.int32).reshape(-1, 4)
    if order == ORDER_FOLDED_ZIGZAG:
        items = []   # lists of tile indices, in generation order of their first tile
        g = 0
        while g < len(tiles):
            e = g
            while e < len(tiles) and tiles[e][:2] == tiles[g][:2]:
                e += 1
            n = e - g
            if causal:
                items += [[g + a, g + n - 1 - a] for a in range(n // 2)]
                if n % 2:
                    items.append([g + n // 2])
            else:
                items += [[g + a] for a in range(n)]
            g = e
        work = [sum(tiles[i][3] for i in it) for it in items]
        ranked = sorted(range(len(items)), key=lambda k: (-work[k], k))
        per_slot = [[] for _ in range(num_slots)]
        for j, k in enumerate(ranked):
            per_slot[_zigzag_rank(j, num_slots)].extend(tiles[i] for i in items[k])
        slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
        flat = []
        for s in range(num_slots):
            flat.extend(per_slot[s])
            slot_ptr[s + 1] = len(flat)
        return slot_ptr, np.asarray(flat, dtype=np.int32).reshape(-1, 4)
    if order == ORDER_ZIGZAG:
        idx = sorted(range(len(tiles)), key=lambda g: (-tiles[g][3], g))
    else:
        idx = list(range(len(tiles)))
    per_slot = [[] for _ in range(num_slots)]
    for j, g in enumerate(idx):
        p, r = divmod(j, num_slots)
        if order == ORDER_ZIGZAG and p % 2 == 1:
            slot = num_slots - 1 - r
        else:
            slot = r
        per_slot[slot].append(tiles[g])
    slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
    flat = []
    for s in range(num_slots):
        flat.extend(per_slot[s])
        slot_ptr[s + 1] = len(flat)
    arr = np.asarray(flat, dtype=np.int32).reshape(-1, 4)
    return slot_ptr, arr


def slot_loads(slot_ptr, tiles, cost=lambda work: work):
    """Sum of per-tile cost in every slot."""
    loads = []
    for s in range(len(slot_ptr) - 1):
        loads.append(sum(cost(int(w)) for w in tiles[slot_ptr[s]:slot_ptr[s + 1], 3]))
    return loads
