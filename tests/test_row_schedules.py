"""Host models of the block-sparse row schedules (no GPU): the index
arithmetic of the XCD-major row order and of the persistent launch's per-XCD
row queues, restated from attn_kernels.hip, checked for the properties the
kernels rely on -- every (head, query block) row is taken exactly once, and
every workgroup of the persistent launch ends."""
import heapq

import numpy as np
import pytest

XCDS = 8


def xcd_major_row(w, bh_total, nb):
    """(flattened head, query block) of workgroup w in the XCD-major order."""
    per = bh_total // XCDS
    qb = nb - 1 - w // bh_total
    local = w % bh_total
    return (local % XCDS) * per + local // XCDS, qb


@pytest.mark.parametrize("bh_total,nb", [(8, 1), (8, 5), (16, 128), (32, 256), (64, 7), (96, 33)])
def test_xcd_major_order_is_a_permutation_with_xcd_ownership(bh_total, nb):
    seen = set()
    for w in range(bh_total * nb):
        bh, qb = xcd_major_row(w, bh_total, nb)
        assert 0 <= bh < bh_total and 0 <= qb < nb and (bh, qb) not in seen
        seen.add((bh, qb))
        # workgroup w runs on XCD w % 8, which owns the heads [x per, (x+1) per)
        x = w % XCDS
        assert x * (bh_total // XCDS) <= bh < (x + 1) * (bh_total // XCDS)
    assert len(seen) == bh_total * nb
    # the longest rows come first
    qbs = [xcd_major_row(w, bh_total, nb)[1] for w in range(bh_total * nb)]
    assert qbs == sorted(qbs, reverse=True)


def rows_h0(y, bh_total):
    return (y * bh_total) // XCDS


def queue_len(y, bh_total, nb):
    return (rows_h0(y + 1, bh_total) - rows_h0(y, bh_total)) * nb


def queue_row(y, j, bh_total, nb):
    h0 = rows_h0(y, bh_total)
    nh = rows_h0(y + 1, bh_total) - h0
    i = j // nh
    return h0 + (j - i * nh), nb - 1 - i


def simulate_persistent(bh_total, nb, slots, cost, seed, steal=True):
    """Event simulation of attn_sparse_rows_kernel: `slots` workgroups per
    XCD, each row taking cost(bh, qb) * (random jitter) time units; claims
    are atomic increments of the per-queue counters (which start at `slots`),
    a dry queue sends the workgroup to the queue with the most rows left."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctr = [slots] * XCDS
    done = {}
    ends = 0
    makespan = 0.0
    events = []
    for wg in range(XCDS * slots):
        x = wg % XCDS
        events.append((0.0, wg, x, wg // XCDS))           # (time, workgroup, queue, row index)
    heapq.heapify(events)
    while events:
        t, wg, y, j = heapq.heappop(events)
        if j >= queue_len(y, bh_total, nb):
            rem = [queue_len(q, bh_total, nb) - ctr[q] for q in range(XCDS)]
            if not steal:
                rem = [r if q == wg % XCDS else 0 for q, r in enumerate(rem)]
            best = max(rem)
            if best <= 0:
                ends += 1
                makespan = max(makespan, t)
                continue
            y = rem.index(best)                             # ties to the lower queue
            j = ctr[y]
            ctr[y] += 1
            heapq.heappush(events, (t + 1e-3, wg, y, j))
            continue
        bh, qb = queue_row(y, j, bh_total, nb)
        assert (bh, qb) not in done, "a row was taken twice"
        done[(bh, qb)] = wg
        nj = ctr[y]                                         # the claim made during the row's last tile
        ctr[y] += 1
        heapq.heappush(events, (t + cost(bh, qb) * rng.uniform(0.5, 1.5), wg, y, nj))
    return done, ends, makespan


@pytest.mark.parametrize("bh_total,nb,slots", [(32, 512, 128), (3, 40, 4), (1, 300, 16), (16, 65, 8), (40, 17, 32)])
def test_persistent_row_queues_take_every_row_once_and_end(bh_total, nb, slots):
    # a mask whose work differs between heads: head h costs (h % 5 + 1) per tile
    cost = lambda bh, qb: (bh % 5 + 1) * (0.1 * qb + 1)
    done, ends, _ = simulate_persistent(bh_total, nb, slots, cost, seed=bh_total * 1000 + nb)
    assert len(done) == bh_total * nb
    assert ends == XCDS * slots


def test_persistent_stealing_balances_the_xcds():
    # one XCD's heads carry 4x the work of the others' heads
    bh_total, nb, slots = 32, 256, 16
    heavy = set(range(rows_h0(0, bh_total), rows_h0(1, bh_total)))
    cost = lambda bh, qb: (4.0 if bh in heavy else 1.0) * (qb + 1)
    done, _, with_steal = simulate_persistent(bh_total, nb, slots, cost, seed=7)
    done_ns, _, without = simulate_persistent(bh_total, nb, slots, cost, seed=7, steal=False)
    assert len(done) == len(done_ns) == bh_total * nb
    assert any(bh in heavy and wg % XCDS != 0 for (bh, qb), wg in done.items())   # other XCDs took its rows
    # balanced, the total work over 8 XCDs would take (4 + 7) / 8 of the heavy
    # XCD's own time; stealing comes within 10% of that
    assert with_steal < 0.6 * without
    assert with_steal < 1.1 * without * (4 + 7) / (8 * 4)


# ---- the XCD-owned key chunks: two launches of attn_sparse_xcd_kernel -------

CHUNK = 128


def xcd_job(x, t, njobs):
    """Job at position t of XCD x's sequence (16 jobs dealt as 0..7, 7..0 over
    each pair of positions), or -1 past its end."""
    base = 2 * XCDS * (t >> 1)
    k = base + 2 * XCDS - 1 - x if t & 1 else base + x
    return k if k < njobs else -1


def xcd_items(x, batch, hkv, group, nb, diag):
    """(batch, query head, query block, chunk) items of XCD x's sequence in one
    launch: the chunks before each row's diagonal chunk (diag=False), or each
    row's diagonal chunk (diag=True)."""
    nch = -(-nb // CHUNK)
    njobs = batch * hkv * nch
    t = 0
    while True:
        job = xcd_job(x, t, njobs)
        if job < 0:
            return
        c, gi = job % nch, job // nch
        b, g = gi // hkv, gi % hkv
        if diag:
            rows = min(nb - c * CHUNK, CHUNK)
            for mi in range(group * rows):          # query block major, ascending, heads in turn
                yield b, g * group + mi % group, c * CHUNK + mi // group, c
        else:
            rows = max(nb - (c + 1) * CHUNK, 0)
            for mi in range(group * rows):          # head major, query block descending
                yield b, g * group + mi // rows, nb - 1 - mi % rows, c
        t += 1


def xcd_slot_base(qb, c):
    k = qb // c
    return qb + c * k * (k - 1) // 2 + k * (qb - k * c) - c


@pytest.mark.parametrize("batch,hkv,group,nb", [(1, 8, 4, 2048), (1, 8, 1, 960), (2, 4, 2, 1000),
                                                (1, 16, 1, 1300), (1, 8, 2, 1290), (3, 8, 1, 1025),
                                                (1, 8, 8, 1000), (2, 3, 2, 1400), (2, 4, 2, 1400)])
def test_xcd_two_launches_cover_every_item_once(batch, hkv, group, nb):
    """The first launch takes exactly the (row, chunk) items before each row's
    diagonal chunk, the second exactly one item per row (its diagonal chunk),
    each once, every XCD's sequence ends, and the partial slots the first
    launch writes are distinct and inside the per-head slot range the second
    launch reads from."""
    hq = hkv * group
    first = [it for x in range(XCDS) for it in xcd_items(x, batch, hkv, group, nb, False)]
    second = [it for x in range(XCDS) for it in xcd_items(x, batch, hkv, group, nb, True)]
    want_first = {(b, h, qb, c) for b in range(batch) for h in range(hq) for qb in range(nb)
                  for c in range(qb // CHUNK)}
    want_second = {(b, h, qb, qb // CHUNK) for b in range(batch) for h in range(hq) for qb in range(nb)}
    assert len(first) == len(set(first)) and set(first) == want_first
    assert len(second) == len(set(second)) and set(second) == want_second
    per_head = xcd_slot_base(nb, CHUNK)
    slots = [(b, h, xcd_slot_base(qb, CHUNK) + c) for b, h, qb, c in first]
    assert len(slots) == len(set(slots))
    assert all(0 <= s < per_head for _, _, s in slots)
    # every slot a diagonal item reads was written by the first launch
    written = set(slots)
    for b, h, qb, c in second:
        assert all((b, h, xcd_slot_base(qb, CHUNK) + cc) in written for cc in range(c))


def test_xcd_first_launch_balanced_at_128k():
    """At 128k with 8 KV groups (the headline layer) every XCD gets chunks c and
    15 - c of each group in the first launch: the same number of items and the
    same number of causal tiles, and in the second launch the same number of
    rows and of partial slots to merge."""
    nb, hkv, group = 2048, 8, 4
    items = [list(xcd_items(x, 1, hkv, group, nb, False)) for x in range(XCDS)]
    assert len({len(i) for i in items}) == 1
    tiles = [sum(min(CHUNK, qb - c * CHUNK) for _, _, qb, c in i) for i in items]
    assert len(set(tiles)) == 1
    diag = [list(xcd_items(x, 1, hkv, group, nb, True)) for x in range(XCDS)]
    assert len({len(d) for d in diag}) == 1
    assert len({sum(c for _, _, _, c in d) for d in diag}) == 1
