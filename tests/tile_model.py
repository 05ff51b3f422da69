"""Host replay of the grouped tile kernel's choice of rows per row tile, so
tests can assert which tile shape a launch runs (the kernel takes this
choice on the device, identically in every workgroup, from the offsets).

It mirrors the launcher and the device code of the 256-row expert
projections:
  * fat tiles (an expert's last remainder of at most 64 rows shared out
    over its other row tiles, up to 320 rows per tile) are allowed from
    K >= 4096;
  * a launch whose tile bound at 256 rows is under 4 rounds of 256 compute
    units picks its rows per row tile per launch, among 256, 224, 192, 160
    and (where allowed) fat tiles, minimising (rounds of tiles) x (32-row
    fragments of the largest tile), ties to fat tiles, then to more rows.
"""
from __future__ import annotations

import numpy as np

BM = 256
FAT_EXTRA = 64
FAT_MIN_K = 4096
ROW_CHOICES = 4
CUS = 256
ADAPT_ROUNDS = 4


def _cdiv(a, b):
    return -(-a // b)


def row_tiles(r: int, tr: int) -> int:
    """Row tiles of a group of r rows at tr rows per tile (tr > BM: fat)."""
    if tr <= BM:
        return _cdiv(r, tr)
    m = _cdiv(r, BM)
    if m > 1 and r - (m - 1) * BM <= tr - BM:
        m -= 1
    return m


def choose_rows(counts, rows: int, K: int, N: int, swiglu: bool):
    """(rows per row tile, tiles, adaptive launch?) for a grouped launch of
    the expert projections.  N: output columns (f for gate/up, d for down);
    rows: the rows argument of the call."""
    counts = np.asarray(counts, np.int64)
    G = counts.size
    bno = 128 if swiglu else 256
    ntiles = _cdiv(N, bno)
    fat_ok = K >= FAT_MIN_K
    FAT = BM + FAT_EXTRA
    bound = (_cdiv(rows, BM) + G) * ntiles
    adapt = bound < ADAPT_ROUNDS * CUS
    if not adapt:
        tr = FAT if fat_ok else BM
    else:
        tot = [sum(_cdiv(int(r), BM - 32 * c) * ntiles for r in counts) for c in range(ROW_CHOICES)]
        maxf = _cdiv(int(counts.max()), 32) if G else 0
        best, best_cost = BM, None
        if fat_ok:
            fat_tiles = sum(row_tiles(int(r), FAT) * ntiles for r in counts if r > 0)
            fat_frags = max([(_cdiv(int(r), 32) + row_tiles(int(r), FAT) - 1) // row_tiles(int(r), FAT)
                             for r in counts if r > 0] or [0])
            best, best_cost = FAT, _cdiv(fat_tiles, CUS) * fat_frags
        for c in range(ROW_CHOICES):
            rc = BM - 32 * c
            cost = _cdiv(tot[c], CUS) * min(rc // 32, maxf)
            if best_cost is None or cost < best_cost:
                best, best_cost = rc, cost
        tr = best
    tiles = sum(row_tiles(int(r), tr) * ntiles for r in counts if r > 0)
    return tr, tiles, adapt
