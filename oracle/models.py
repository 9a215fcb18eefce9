"""Analytic models from gpu-kernels-explained "Split-K, streams and overlap"
(test infrastructure; they give the split policy its rationale).

``splitk_wave_model`` -- section Maths, "Split-K": with s slices there are
tiles*s blocks and ceil(tiles*s / SMs) waves; each block does 2*b_m*b_n*(k/s)
flops, so the compute time is waves times one block's flops at one SM's share
of the peak; for s > 1 the second pass adds 2*4*m*n*s bytes (the fp32 partials
written and read back) at the memory bandwidth. With s = 1 there is no second
pass. The page prints this model's output for a 512 x 512 x 16384 BF16 GEMM
on an A100 (table "Split-K on the A100"); the model's two machine constants are
not printed there -- the A100's public dense BF16 peak (312 TFLOP/s) and HBM
bandwidth (1555 GB/s) reproduce every row to the table's 0.1 us precision.

``overlap_schedule`` -- section Maths, "Overlap": three engines (load, compute,
store) each handle one tile at a time, in tile order; tile i's load starts
after the previous load and after tile (i - b)'s compute has freed its buffer
(b buffers); a tile's compute starts after its load and the previous compute;
its store after its compute and the previous store. The total time is the end
of the last store.
"""
import math


def splitk_wave_model(s, *, m=512, n=512, k=16384, tile_m=128, tile_n=128, sms=108,
                      peak_flops=312e12, bandwidth=1555e9):
    """Returns dict(blocks, waves, time_s, compute_s, reduce_s) for split count s."""
    tiles = math.ceil(m / tile_m) * math.ceil(n / tile_n)
    blocks = tiles * s
    waves = math.ceil(blocks / sms)
    block_flops = 2.0 * tile_m * tile_n * (k / s)
    compute = waves * block_flops / (peak_flops / sms)
    reduce = (2 * 4 * m * n * s) / bandwidth if s > 1 else 0.0
    return dict(tiles=tiles, blocks=blocks, waves=waves, compute_s=compute, reduce_s=reduce,
                time_s=compute + reduce)


def idle_fraction(blocks, sms):
    """Fraction of SMs with no block in a single under-filled wave."""
    return 1.0 - min(blocks, sms) / sms


def overlap_schedule(n_tiles, t_load, t_comp, t_store, buffers):
    """Event-by-event schedule; returns the time the last store ends."""
    load_end, comp_end, store_end = [], [], []
    for i in range(n_tiles):
        ls = load_end[i - 1] if i > 0 else 0.0
        if i >= buffers and comp_end[i - buffers] > ls:
            ls = comp_end[i - buffers]
        load_end.append(ls + t_load)
        cs = max(load_end[i], comp_end[i - 1] if i > 0 else 0.0)
        comp_end.append(cs + t_comp)
        ss = max(comp_end[i], store_end[i - 1] if i > 0 else 0.0)
        store_end.append(ss + t_store)
    return store_end[-1] if store_end else 0.0


def overlap_closed_form(n_tiles, t_load, t_comp, t_store):
    """The page's approximation for b >= 2: t_load + n*max(times) + t_store."""
    return t_load + n_tiles * max(t_load, t_comp, t_store) + t_store


def single_buffer_closed_form(n_tiles, t_load, t_comp, t_store):
    """The page's exact b = 1 time: n*(t_load + t_comp) + t_store."""
    return n_tiles * (t_load + t_comp) + t_store
