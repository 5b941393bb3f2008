"""Launch configuration of each workload: tile shape and micro-batch chunk
sizes.  Used by the benchmark and by the parity tests, so that the tests
check exactly the configuration that is timed."""

# (tile_m, tile_n) per workload key of inputs.CONFIGS
# chosen by the steady-state pipelined time of each candidate on one MI355X
# (C2: 128x64 78 us vs 128x128 94 us; C4: 128x128 537 us vs 256x128 548 us;
# C5: 128x128 and 256x128 both ~572 us)
TILES = {
    "c1": (64, 64),
    "c2": (128, 64),
    "c3": (256, 256),
    "c4": (128, 128),
    "c5": (128, 128),
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
