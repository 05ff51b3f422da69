"""The host replay of the tile kernel's rows-per-tile choice on shapes whose
outcome is known from the kernel's design (CPU only)."""
from tests.tile_model import choose_rows, row_tiles


def test_row_tiles():
    assert row_tiles(1072, 256) == 5
    assert row_tiles(1072, 320) == 4          # 48-row remainder folded
    assert row_tiles(1100, 320) == 5          # 76 rows: too many to fold
    assert row_tiles(300, 320) == 1
    assert row_tiles(256, 320) == 1


def test_long_launches_keep_their_tiles():
    # 256 experts, many rows: more than 4 rounds at 256 rows -> no per-launch choice
    tr, tiles, adapt = choose_rows([512] * 256, 131072, 7168, 2048, swiglu=True)
    assert not adapt and tr == 320
    tr, tiles, adapt = choose_rows([512] * 256, 131072, 2048, 7168, swiglu=False)
    assert not adapt and tr == 256


def test_short_launch_prefers_fat_tiles():
    # 8 experts of 1072 rows at K = 4096: 256 fat tiles in one round
    assert choose_rows([1072] * 8, 8576, 4096, 2048, swiglu=False) == (320, 256, True)
    # below K = 4096 fat tiles are not allowed: 160-row tiles (7 per expert)
    tr, tiles, adapt = choose_rows([1072] * 8, 8576, 2048, 2048, swiglu=False)
    assert adapt and tr == 160 and tiles == 8 * 7 * 8
