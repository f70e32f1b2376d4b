"""The grouped FFN's tile-schedule codes, on the host (no GPU): the M-tile
count the library's m_tiles gives every expert row count is checked against
a walk that lays the tiles over the rows one by one (step rows per tile, a
remainder of at most `extra` rows joining the last full tile), the two-class
codes keep exactly the experts of their class, every expert of the few-row
class takes at most one tile (the bound the side-stream launch's grid is
sized by), and the library picks two classes only for bf16 layers of at
least 64 experts on tall tiles without a split down projection."""

import os
import shutil
import subprocess

import pytest

from mixture_experts_layer_wavefront_amd import build as Bd

HERE = os.path.dirname(os.path.abspath(__file__))


def _walk(rows, step, extra):
    """Tiles laid over `rows` rows: each takes `step` rows, except that the
    last full tile also takes a remainder of at most `extra` rows."""
    tiles, start = [], 0
    while start < rows:
        end = min(start + step, rows)
        if end - start == step and 0 < rows - end <= extra:
            end = rows
        tiles.append((start, end))
        start = end
    return tiles


@pytest.fixture(scope="module")
def schedule_output(tmp_path_factory):
    if not os.path.exists(Bd.LIB):
        pytest.skip("library not built")
    try:
        hipcc = Bd._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("tiles") / "tile_schedule")
    cmd = [hipcc, "-std=c++17", "-O1", "-x", "hip", f"--offload-arch={Bd.ARCH}",
           "-I", Bd.INCLUDE, "-I", Bd.CSRC, os.path.join(HERE, "host", "tile_schedule.cpp"),
           "-o", exe, "-L", Bd.PKG, "-lmoe_mi355x", f"-Wl,-rpath,{Bd.PKG}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    shapes, codes, class_rows = [], {}, None
    for line in out.splitlines():
        f = line.split()
        if f[0] == "shape":
            shapes.append((tuple(int(x) for x in f[1:7]), int(f[8]), int(f[10]), int(f[12]),
                           int(f[14])))
        elif f[0] == "class_rows":
            class_rows = int(f[1])
        elif f[0] == "code":
            codes[int(f[1].rstrip(":"))] = [int(x) for x in f[2:]]
    return shapes, codes, class_rows


def _decode(code):
    return code & 0xFFFF, (code >> 16) & 0xFF, (code >> 24) & 3


def test_m_tiles_matches_the_tile_walk(schedule_output):
    _, codes, class_rows = schedule_output
    assert class_rows == 160
    for code, counts in codes.items():
        step, extra, cls = _decode(code)
        for rows, n in enumerate(counts):
            in_class = {0: True, 1: rows <= class_rows, 2: rows > class_rows}[cls]
            tiles = _walk(rows, step, extra) if in_class else []
            assert n == len(tiles), (code, rows, n, tiles)
            # the tiles cover the rows once; none exceeds step + extra rows
            assert sum(e - s for s, e in tiles) == (rows if in_class else 0)
            assert all(e - s <= step + extra for s, e in tiles)


def test_two_class_codes(schedule_output):
    shapes, codes, class_rows = schedule_output
    by_shape = {s[0]: s[1:] for s in shapes}
    # (bf16, fp8, E, mean rows, d, d_ff) -> two classes?
    assert by_shape[(1, 0, 128, 1024, 2048, 768)][0] == 1
    assert by_shape[(1, 0, 64, 257, 256, 192)][0] == 1
    for key in [(1, 0, 32, 1024, 2880, 2880), (1, 0, 8, 1024, 4096, 14336),
                (1, 0, 256, 128, 7168, 2048), (1, 0, 64, 256, 256, 192),
                (1, 1, 128, 1024, 2048, 768), (0, 0, 128, 1024, 2048, 768),
                (1, 0, 16, 375, 264, 2112)]:
        assert by_shape[key][0] == 0, key
        assert by_shape[key][2] == 0, key   # no second schedule
    assert by_shape[(1, 0, 16, 375, 264, 2112)][3] == 1  # split: one class
    two, code, code2, _ = by_shape[(1, 0, 128, 1024, 2048, 768)]
    small, large = codes[code], codes[code2]
    for rows in range(len(small)):
        if rows == 0:
            assert small[rows] == 0 and large[rows] == 0
        elif rows <= class_rows:
            assert small[rows] == 1 and large[rows] == 0, rows
        else:
            assert small[rows] == 0 and large[rows] >= 1, rows
    # the large class keeps the one-class tall schedule for its experts
    one_class_code = by_shape[(1, 0, 32, 1024, 2880, 2880)][1]
    tall = codes[one_class_code]
    assert all(large[r] == tall[r] for r in range(class_rows + 1, len(tall)))
