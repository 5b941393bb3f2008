"""Launch configuration of each workload: tile shape and micro-batch chunk
sizes.  Used by the benchmark and by the parity tests, so that the tests
check exactly the configuration that is timed."""

# (tile_m, tile_n) per workload key of inputs.CONFIGS, chosen by the
# pipelined time of each candidate, interleaved on one MI355X (microseconds):
#   C2: 64x128 (four stages, 8 waves as 2 x 4, one workgroup per CU,
#       unsplit) 54.7; the same on 4 waves 55-58;
#       128x64 (three stages, two per CU, split 2) 59-61; 64x128 on three
#       stages 61; 64x128 on four stages split 2 78; 128x128 72-77; 64x64
#       64-75; 64x256 75; 256x64 81; 256x128 98; 128x256 99; 256x256 115
#   C3: 256x256 395-428; 256x128 517; 128x256 521
#   C4: 128x128 514-524; 256x128 on 8 waves (4 x 2) 514 (sequential 507
#       there, 521 for 128x128); 256x128 on 4 waves 525-545 (16x16x32
#       blocks, 8 waves as 2 x 4: 554-560);
#       256x256 539-547 (split 2; 516-525 with the pipelined split-K sum,
#       level with 128x128 then)
#   C5: 256x128 (8 waves as 4 x 2, three stages, one workgroup per CU)
#       280-281; 128x256 (same) 282-284; 128x128 303-313; 256x128 on
#       4 waves 320; 256x64 376; 64x256 381
TILES = {
    "c1": (64, 64),
    "c2": (64, 128),
    "c3": (256, 256),
    "c4": (128, 128),
    "c5": (256, 128),
}

# rows per chunk swept by the micro-batched baseline (each a multiple of tile_m
# that divides M and leaves at least two chunks)
def chunk_sweep(M: int, tile_m: int):
    out = []
    m = tile_m
    while m < M:
        if M % m == 0:
            out.append(m)
        m *= 2
    return out


def microbatch_tile(M: int, tile):
    """Tile of the micro-batched baseline: the timed tile, or, where that
    tile leaves no two chunks (tile_m = M, as with 256-row tiles on a 256-row
    batch), the tile with tile_m halved until it does."""
    bm, bn = tile
    while not chunk_sweep(M, bm) and bm > 64:
        bm //= 2
    return (bm, bn)

