"""A second, independent implementation of capacity routing (test pin only).

The oracle walks the slots one at a time.  This version reaches the same
assignment by a different route: for each pass it iterates, in parallel over
tokens, a threshold tau[e] per expert (the index of the last token that
expert e can still accept).  Every token proposes to its best expert e that
it does not hold and for which token <= tau[e]; tau[e] then becomes the
index of the (room_e)-th proposer of e.  tau only decreases, so the
iteration stops, and its fixed point is the serial first-come assignment
(deferred acceptance with one common priority order, the token index).

It shares no code with oracle/: the ranking is recomputed here with
Python's sort.
"""
from __future__ import annotations

import numpy as np

INF = 1 << 60


def _ranking(z):
    T, N = z.shape
    return [sorted(range(N), key=lambda e, row=z[t]: (-float(row[e]), e)) for t in range(T)]


def capacity_route_fixed_point(z, k: int, C: int):
    z = np.asarray(z, dtype=np.float64)
    T, N = z.shape
    order = _ranking(z)
    fill = np.zeros(N, dtype=np.int64)
    idx = np.full((T, k), -1, dtype=np.int64)
    for j in range(k):
        room = C - fill
        tau = np.full(N, INF, dtype=np.int64)
        while True:
            choice = np.full(T, -1, dtype=np.int64)
            for t in range(T):
                held = set(idx[t, :j].tolist())
                for e in order[t]:
                    if e in held or room[e] <= 0 or t > tau[e]:
                        continue
                    choice[t] = e
                    break
            new_tau = np.full(N, INF, dtype=np.int64)
            for e in range(N):
                takers = np.nonzero(choice == e)[0]   # ascending token ids
                if room[e] > 0 and takers.size >= room[e]:
                    new_tau[e] = takers[room[e] - 1]
            if np.array_equal(new_tau, tau):
                break
            tau = new_tau
        idx[:, j] = choice
        for e in choice[choice >= 0]:
            fill[e] += 1
    return idx, fill
