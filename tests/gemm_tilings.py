"""Shapes that reach every tiling of the large-M path: (bits, waves, tile
rows, tile columns, K split?) -> (m, n, k) with ragged M, N and K; and the
cuts of the stream-K path: (bits, tile rows, tile columns, runs inside
tiles?) -> (m, n, k), with runs that each lie inside one tile (4 or 16 runs
sharing a tile) and runs that cross tile ends (a run's two segments, three
or more runs sharing a tile).  The plan of each shape is checked on the host (test_boundary.py),
the results on the GPU (test_gemm_tiles_gpu.py)."""

TILINGS = [
    # (bits, waves, tile_m, tile_n, split, (m, n, k))
    (4, 4, 64, 256, False, (130, 32772, 128)),
    (4, 4, 64, 256, True, (257, 8200, 4096)),
    (4, 8, 128, 128, False, (97, 136, 128)),
    (4, 8, 128, 128, True, (97, 136, 640)),
    (4, 8, 128, 256, False, (257, 16424, 128)),
    (4, 8, 128, 256, True, (97, 16424, 2176)),
    (4, 8, 256, 128, False, (130, 16424, 128)),
    (4, 8, 256, 128, True, (130, 2056, 4096)),
    (4, 8, 256, 256, False, (1000, 8200, 128)),
    (4, 8, 256, 256, True, (130, 16424, 4096)),
    (8, 8, 128, 128, False, (97, 136, 128)),
    (8, 8, 128, 128, True, (97, 136, 640)),
    (8, 8, 128, 256, False, (257, 16424, 128)),
    (8, 8, 128, 256, True, (97, 16424, 2176)),
    (8, 8, 256, 128, False, (130, 16424, 128)),
    (8, 8, 256, 128, True, (130, 2056, 4096)),
    (8, 8, 256, 256, False, (130, 32772, 128)),
    (8, 8, 256, 256, True, (257, 8200, 4096)),
]


STREAMK_TILINGS = [
    # (bits, tile_m, tile_n, runs inside tiles?, (m, n, k))
    (4, 128, 128, True, (1000, 136, 2048)),
    (4, 256, 128, True, (257, 4000, 2048)),
    (4, 128, 128, False, (130, 4104, 512)),
    (4, 128, 256, False, (257, 16424, 640)),
    (4, 256, 128, False, (130, 16424, 384)),
    (8, 128, 128, True, (1000, 136, 2048)),
    (8, 256, 128, True, (257, 4000, 2048)),
    (8, 128, 128, False, (130, 4104, 512)),
    (8, 128, 256, False, (257, 16424, 640)),
    (8, 256, 128, False, (130, 16424, 384)),
]


def streamk_id(t):
    bits, tm, tn, inside, (m, n, k) = t
    return f"int{bits}_{tm}x{tn}_{'inside' if inside else 'crossing'}_m{m}_n{n}_k{k}"


def tiling_id(t):
    bits, waves, tm, tn, split, (m, n, k) = t
    return f"int{bits}_{waves}w_{tm}x{tn}_{'split' if split else 'unsplit'}_m{m}_n{n}_k{k}"
