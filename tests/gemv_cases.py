"""Shapes of the GEMV parity cases, shared by the GPU parity tests and by the
CPU test that checks that every GEMV kernel instance a benchmarked workload
launches is run by at least one of them. Shapes only: no arithmetic of the
method here."""

Q4_0, Q8_0, Q4_K, Q4_0_F16 = 1, 2, 3, 4
TYPES = [Q4_0, Q8_0, Q4_K, Q4_0_F16]

# qblk_gemv against the oracle, every type: (n, k, batch)
GEMV_RANDOM = [(37, 1024, 1), (300, 4096, 1), (129, 2304, 4), (64, 256, 8), (70, 512, 64),
               (3100, 512, 2), (16400, 512, 5),
               # a single row and two rows: one wave, most lanes past the last row
               (1, 256, 1), (2, 512, 3),
               # Q4_K's matrix-core kernel (2-8 rows, k a multiple of 2048): one
               # 2048-element chunk with a ragged last tile, and fewer rows than a tile
               (1000, 2048, 3), (5, 4096, 4)]

# Q4_K's matrix-core kernel with exact fp32 arithmetic: (n, k, batch)
GEMV_RING_EXACT = [(67, 4096, 2), (67, 4096, 3), (67, 4096, 4), (16, 2048, 4), (67, 4096, 5), (16, 2048, 8),
                   # more than 512 tiles of one chunk (the one-tile kernel)
                   (8208, 2048, 2),
                   # more than 512 tiles of two chunks or more (the tile-walking grid): a
                   # ragged last tile, and 1025 tiles, so that one workgroup takes three and
                   # the others two, at 3, 4, 6 and 8 rows
                   (8200, 4096, 3), (16400, 4096, 4), (8200, 4096, 6), (16400, 4096, 8)]

# qblk_gemv with exact fp32 arithmetic, every type: batch (n = 67, k = 2304 / 2336)
GEMV_EXACT_BATCH = [1, 3, 8, 11]

# qblk_gemv at the configured sizes, sampled rows: (name, workload, type, n, k)
GEMV_FULL_SIZE = [
    ("Q4_0 4096x4096", 1, Q4_0, 4096, 4096),
    ("Q8_0 14336x4096", 2, Q8_0, 14336, 4096),
    ("Q4_K q 4096x4096", 3, Q4_K, 4096, 4096),
    ("Q4_K k 1024x4096", 3, Q4_K, 1024, 4096),
    ("Q4_K gate 14336x4096", 3, Q4_K, 14336, 4096),
    ("Q4_K down 4096x14336", 3, Q4_K, 4096, 14336),
]

# qblk_gemv, 70B-shaped Q4_K matrices, sampled rows: (name, n, k) x batch
GEMV_70B = [("q", 8192, 8192), ("gate", 28672, 8192), ("down", 8192, 28672)]
GEMV_70B_BATCH = [1, 4, 8]

# qblk_gemm at m rows of Q4_K 14336 x 4096; for m <= 64 qblk_gemv on the same inputs
GEMM_PREFILL_M = [512, 1, 8, 64]

# qblk_gemv_f32 bitwise against qblk_quantize_act + qblk_gemv, and against
# the oracle on sampled rows, every type: (n, k, batch)
GEMV_F32 = [(37, 1024, 1), (300, 4096, 3), (4100, 2304, 1), (9000, 8192, 1), (129, 4096, 6),
            (70, 256, 8), (2000, 28672, 1), (17000, 4096, 1), (8200, 16384, 1), (16400, 4096, 3),
            (16384, 2048, 8), (5000, 28672, 4)]

# qblk_gemv_f32 with the in-launch handoff and a reused workspace, every type
GEMV_F32_IN_LAUNCH = [(9000, 8192, 1), (20000, 4096, 1), (8192, 28672, 1), (4096, 14336, 1),
                      (4096, 4096, 1), (1024, 4096, 2), (9000, 4096, 4), (16400, 2304, 3),
                      (3, 1 << 24, 1), (3, 1 << 24, 4),
                      # the row-group classes of the 70B-shaped decode at k = 8192
                      # (Q4_K: the matrix-core kernels; the other types: 8 rows per
                      # wave with the activations in LDS and 4 rows per wave), and
                      # their batch-1 controls
                      (16400, 8192, 4), (9000, 8192, 4), (16400, 8192, 1),
                      # the same at 2 and 8 rows, with a ragged last workgroup at 6200 rows
                      (6200, 8192, 2), (8192, 8192, 8),
                      # Q4_K's 8-wave dot4 workgroups (6k-8k rows, k above 4096 but not a
                      # multiple of 2048, batch 2-8)
                      (6200, 6400, 2), (8192, 6400, 8)]

# qblk_gemv_f32, Q4_K on the tile-walking matrix-core kernel with the
# in-launch handoff: 513-750 tiles of 2-5 chunks (so that some workgroups of
# the 512-workgroup grid take two tiles), every batch 2-8
GEMV_F32_RING_TILES = [(8200, 4096, 2), (9000, 6144, 3), (8208, 8192, 4), (12000, 10240, 5),
                  (8200, 4096, 6), (9000, 4096, 7), (10000, 8192, 8)]
# ... and with exact fp32 arithmetic (power-of-two scales)
GEMV_F32_RING_TILES_EXACT = [(8200, 4096, 3), (9000, 6144, 8)]

# qblk_gemv_f32 at the 70B-shaped decode's own matrices (q/k/v and gate/up
# concatenated by rows), Q4_K, sampled rows: (name, n, k) x batch
GEMV_F32_70B = [("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192),
                ("down", 8192, 28672),
                # one GPU's share of the same layer split over 8 GPUs
                ("qkv_tp8", 1280, 8192), ("o_tp8", 8192, 1024), ("gate_up_tp8", 7168, 8192),
                ("down_tp8", 8192, 3584)]
GEMV_F32_70B_BATCH = [1, 4]


def covered():
    """(type, n, k, batch, fused) of every GEMV call the parity tests make
    and check (qblk_gemv_f32 cases also run qblk_gemv on the same shape)."""
    out = set()
    for t in TYPES:
        for n, k, b in GEMV_RANDOM:
            if t != Q4_K or k % 256 == 0:
                out.add((t, n, k, b, False))
        for b in GEMV_EXACT_BATCH:
            out.add((t, 67, 2304 if t == Q4_K else 2336, b, False))
    for n, k, b in GEMV_RING_EXACT:
        out.add((Q4_K, n, k, b, False))
    for t in TYPES:
        for n, k, b in GEMV_F32 + GEMV_F32_IN_LAUNCH:
            if t != Q4_K or k % 256 == 0:
                out.add((t, n, k, b, True))
                out.add((t, n, k, b, False))
    for _, _, t, n, k in GEMV_FULL_SIZE:
        out.add((t, n, k, 1, False))
    for _, n, k in GEMV_70B:
        for b in GEMV_70B_BATCH:
            out.add((Q4_K, n, k, b, False))
    for m in GEMM_PREFILL_M:
        if m <= 64:
            out.add((Q4_K, 14336, 4096, m, False))
    for n, k, b in GEMV_F32_RING_TILES + GEMV_F32_RING_TILES_EXACT:
        out.add((Q4_K, n, k, b, True))
        out.add((Q4_K, n, k, b, False))
    for _, n, k in GEMV_F32_70B:
        for b in GEMV_F32_70B_BATCH:
            out.add((Q4_K, n, k, b, True))
            out.add((Q4_K, n, k, b, False))
    return out
