"""The occupancy split rule, in its plain form (test infrastructure).

tiny-llm "Week 2 Day 7: Split-K Prefill", Task 3 ("Choose Partitions From
Occupancy") states the rule in that page's own letters, where the output width
is called K and the reduction length N. In the notation used everywhere here
(A[M,K], W[N,K], C[M,N], reduction length K, G = K/128 groups) it reads:

    base  = ceil(M / tile_m) * ceil(N / tile_n)        (output tiles, 32 x 32 on the page)
    s     = min(cap, floor(target / base), G)           (cap 16, target 320 on the page)
    while G is not a multiple of s: s -= 1
    s <= 1 -> the unsplit kernel

The page's "N / 128" is the group count G. ``min_k_per_split`` generalises it:
each partition must cover at least that many K values, i.e. s <= K // min_k; the
page's rule is min_k = 128 (one group). The split can never exceed G, because
partitions are equal and group aligned (Task 2).
"""

PAGE_PRESET = dict(tile_m=32, tile_n=32, target=320, cap=16, min_k_per_split=128)


def _ceil_div(a, b):
    return -(-a // b)


def base_tiles(M, N, tile_m, tile_n):
    """Output tiles of the unsplit grid."""
    return _ceil_div(M, tile_m) * _ceil_div(N, tile_n)


def split_count(M, N, K, tile_m=32, tile_n=32, target=320, cap=16, min_k_per_split=128,
                group=128):
    """Split count chosen by the occupancy rule; 1 means the unsplit kernel."""
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    base = base_tiles(M, N, tile_m, tile_n)
    s = min(cap, target // base, G, K // min_k_per_split)
    while s > 1 and G % s != 0:
        s -= 1
    return max(s, 1)
