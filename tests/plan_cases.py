"""Shapes that select every tiling of the lifted large-batch product
(LQ_ALGO_MFMA_LARGE): (N, L, B, z dtype, panels per wavefront, 16-row batch
tiles per workgroup). The CPU test asserts the plan each shape gets through
lq_sign_gemm_plan; the GPU test compares each with the oracle.

The plan takes 4 panels x 8 batch tiles for bf16 z when that still gives
>= 512 workgroups; else up to 4 batch tiles (bf16 z; 2 for fp32 z, whose two
bf16 planes would not fit LDS otherwise; 1 at B <= 16), with the most panels
per wavefront (8, 4, 2) that keeps >= 512 workgroups, or, with 4 batch tiles,
2 if the reduction split still gives >= 256. L is kept short where N is
large (one or two full tiles and a tail) so that the oracle stays cheap.
"""
LARGE_PLAN_CASES = [
    # bf16 z
    (8192, 1544, 2048, "bf16", 4, 8),
    (131072, 1032, 80, "bf16", 8, 4),
    (8192, 1032, 1024, "bf16", 4, 4),
    (65536, 1032, 64, "bf16", 2, 4),
    (1024, 1544, 64, "bf16", 1, 4),
    (131072, 520, 48, "bf16", 8, 2),
    (65536, 520, 48, "bf16", 4, 2),
    (32768, 520, 48, "bf16", 2, 2),
    (1024, 1544, 48, "bf16", 1, 2),
    (262144, 520, 16, "bf16", 8, 1),
    (131072, 520, 8, "bf16", 4, 1),
    (65536, 520, 3, "bf16", 2, 1),
    (256, 1544, 1, "bf16", 1, 1),
    # fp32 z (a bf16 hi + lo pair)
    (65536, 520, 128, "f32", 8, 2),
    (32768, 520, 128, "f32", 4, 2),
    (16384, 520, 128, "f32", 2, 2),
    (1024, 1544, 200, "f32", 1, 2),
    (262144, 520, 1, "f32", 8, 1),
    (131072, 520, 2, "f32", 4, 1),
    (65536, 520, 16, "f32", 2, 1),
    (256, 1544, 4, "f32", 1, 1),
]


def case_id(c):
    N, L, B, zt, pw, jb = c
    return f"N{N}-L{L}-B{B}-{zt}-pw{pw}-jb{jb}"


# Shapes with too few panel and batch groups to fill the chip, on which the
# plan splits the reduction into ranges of >= 8 tiles (as many as keep the
# workgroups within 512): (N, L, B, z dtype, panels per wavefront, batch
# tiles, ranges).
LARGE_SPLIT_CASES = [
    (1024, 8200, 64, "bf16", 1, 4, 2),       # 16 workgroups, 17 tiles (ragged)
    (2048, 65536, 64, "bf16", 2, 4, 16),     # 2 panels per wavefront: 16 x 16 ranges
    (512, 40000, 48, "bf16", 1, 2, 9),       # 16 workgroups, 79 tiles
    (256, 20000, 200, "f32", 1, 2, 5),       # 28 workgroups, 40 tiles
]


def split_case_id(c):
    N, L, B, zt, pw, jb, ks = c
    return f"N{N}-L{L}-B{B}-{zt}-pw{pw}-jb{jb}-k{ks}"
