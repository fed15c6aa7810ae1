"""The LDS chunk swizzles of the attention and weight-only kernels put the 64 lanes of one
fragment read on distinct 16-byte bank groups, whichever of 16, 32 or 64 lanes the LDS serves per
pass.  Lane l reads row n = l % 16 of the fragment, chunk c(l) of that row; the position of a lane
is its byte address modulo the pass window, in 16-byte units.  (CPU check of the index formulas
the kernels use.)"""


def distinct(positions):
    return len(set(positions)) == len(positions)


def check(pos):
    """pos(n, g) -> 16-byte unit address for row n (0..15), lane group g (0..3)."""
    for window in (16, 32, 64):                # 256, 512, 1024 bytes
        lanes_per_pass = window
        groups = lanes_per_pass // 16
        for g0 in range(0, 4, groups):
            assert distinct([pos(n, g) % window for g in range(g0, g0 + groups) for n in range(16)])


def test_attention_k_swizzle():
    """K tile rows of 512 bytes (32 chunks); K step kk reads chunk 4 kk + g."""
    ksw = lambda n: 4 * (n >> 1) + 2 * (n & 1) + ((n >> 3) & 1)
    for kk in range(8):
        check(lambda n, g: n * 32 + ((4 * kk + g) ^ ksw(n)))


def test_attention_vt_swizzle():
    """V^T tile rows of 64 bytes (4 chunks); lane group g reads chunk g."""
    check(lambda n, g: n * 4 + (g ^ ((n >> 2) & 3)))


def test_weight_only_token_swizzle():
    """Token tile rows of 256 bytes (16 chunks); K step s reads chunk 4 g + s."""
    rot4 = lambda n: ((n & 3) << 2) | ((n >> 2) & 3)
    for s in range(4):
        check(lambda n, g: n * 16 + ((4 * g + s) ^ rot4(n)))


def test_plain_xor_fails_for_wide_passes():
    """The plain XOR swizzle (c ^ n) that the weight-only kernel first used is conflict-free only
    for 16-lane passes; its measured bank conflicts are what the rotated form removed."""
    import pytest
    for s in range(4):
        pos = lambda n, g: n * 16 + ((4 * g + s) ^ n)
        assert distinct([pos(n, 0) % 16 for n in range(16)])
        with pytest.raises(AssertionError):
            check(pos)
