"""Oracle for the 128-aligned compensation planner.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests and the
benchmark's CPU leg use it; the library's planner shares no code with it.

Source: the DeepEP compensation PR (Python section) names a water-filling
chunk-migration planner with expert-affinity batching, a makespan guard, a
cost-aware no-op and 128-aligned chunks, and reports ~99 % of the ideal bound;
the TEMPO summary (section 2) gives the tile-aware cost model: an expert's
time on a device is an activation floor plus a cost per 128-row M-tile.  The
pages give no algorithm listing, so the steps below are one plain reading of
those features; the library's C++ planner must reproduce them exactly.

Model (integer cost units, so both implementations agree exactly):
  ranks r = 0..ws-1; expert e lives on rank e // L (L = E / ws);
  assign[r][e] = rows of expert e computed on rank r (initially all on e's
  home rank); load(r) = sum over e with assign[r][e] > 0 of
  activation + tile * ceil(assign[r][e] / 128).
  ideal = ceil(sum_r load0(r) / ws)  (perfect balance, no extra activations).

Step (repeated while fewer than max_moves moves):
  src = most loaded rank, dst = least loaded rank (ties: lowest index);
  stop when load(src) - load(dst) <= tile;
  for every expert e with m_max = assign[src][e] // 128 >= 1 whole chunks,
  moving m chunks (1 <= m <= m_max) of 128 rows gives
    src' = load(src) - m*tile - (activation if the move empties e on src)
    dst' = load(dst) + m*tile + (activation if e is new on dst);
  candidate m values are floor/ceil of (load(src) - load(dst) - new_act) /
  (2*tile) clipped to [1, m_max], and m_max itself; a move is admissible only
  if dst' < load(src) (makespan guard); the chosen move minimises
  (max(src', dst'), e not already on dst, e, m) lexicographically
  (expert-affinity: experts the receiver already computes win ties);
  stop when no move is admissible.
Cost-aware no-op: if makespan_before - makespan_after < min_gain, the plan
is discarded (no moves).

Termination: a move replaces (load(src), load(dst)) by two values both below
the old maximum, so the load vector sorted in descending order strictly
decreases lexicographically; no plan repeats, and max_moves caps the count.
"""

from __future__ import annotations

CHUNK = 128


def _tiles(rows: int) -> int:
    return -(-rows // CHUNK)


def plan(counts, ws: int, tile: int, activation: int, min_gain: int = 0, max_moves: int = 1024):
    """Returns dict(moves=[(expert, src, dst, rows)], loads=[...], before=int,
    after=int, ideal=int)."""
    counts = [int(c) for c in counts]
    e_n = len(counts)
    if ws < 1 or e_n % ws != 0 or tile <= 0 or activation < 0 or max_moves < 0:
        raise ValueError("invalid planner arguments")
    per = e_n // ws
    assign = [[0] * e_n for _ in range(ws)]
    for e, c in enumerate(counts):
        assign[e // per][e] = c

    def load(r):
        return sum(activation + tile * _tiles(a) for a in assign[r] if a > 0)

    loads = [load(r) for r in range(ws)]
    loads0 = list(loads)
    before = max(loads)
    ideal = -(-sum(loads) // ws)
    moves = []
    while len(moves) < max_moves:
        src = max(range(ws), key=lambda r: (loads[r], -r))
        dst = min(range(ws), key=lambda r: (loads[r], r))
        ls, ld = loads[src], loads[dst]
        if ls - ld <= tile:
            break
        best = None
        for e in range(e_n):
            a = assign[src][e]
            m_max = a // CHUNK
            if m_max < 1:
                continue
            on_dst = assign[dst][e] > 0
            new_act = 0 if on_dst else activation
            target = ls - ld - new_act
            cands = {m_max}
            if target > 0:
                q = target // (2 * tile)
                cands |= {q, q + 1}
            for m in sorted(cands):
                if m < 1 or m > m_max:
                    continue
                empties = (m * CHUNK == a)
                s_new = ls - m * tile - (activation if empties else 0)
                d_new = ld + m * tile + new_act
                if d_new >= ls:
                    continue
                key = (max(s_new, d_new), 0 if on_dst else 1, e, m)
                if best is None or key < best[0]:
                    best = (key, e, m, s_new, d_new)
        if best is None:
            break
        _, e, m, s_new, d_new = best
        rows = m * CHUNK
        assign[src][e] -= rows
        assign[dst][e] += rows
        loads[src], loads[dst] = s_new, d_new
        moves.append((e, src, dst, rows))
    after = max(loads)
    if before - after < min_gain:
        moves, loads, after = [], loads0, before
    return {"moves": moves, "loads": loads, "before": before, "after": after, "ideal": ideal}
