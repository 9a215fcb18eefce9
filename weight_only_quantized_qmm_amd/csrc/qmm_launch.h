// qmm_launch.h -- internal interface between the C-ABI host code (qmm_api.cpp)
// and the gfx950 kernels (*.hip). Not installed; the public ABI is include/qmm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace qmm_impl {

// Which W4A16 kernel runs an M-row problem, and the output tile of one workgroup.
//   SKINNY (M <= 64) : a (16*mt) x 32 tile, up to 16 waves splitting its reduction;
//   NARROW (M <= 128): 4 waves side by side along N, each 16*ns columns x 16*mt rows;
//   WIDE   (M > 128) : a 256 x 128 tile.
enum W4A16Kind { W4A16_SKINNY = 0, W4A16_NARROW = 1, W4A16_WIDE = 2 };

struct W4A16Tile {
    W4A16Kind kind;
    int mt;  // 16-row MFMA subtiles per block (SKINNY: 1, 2, 4; NARROW: 8)
    int ns;  // 16-column MFMA subtiles per wave (NARROW) or per block (SKINNY: 2)
    int block_m() const { return kind == W4A16_WIDE ? 256 : 16 * mt; }
    int block_n() const { return kind == W4A16_WIDE ? 128 : kind == W4A16_SKINNY ? 16 * ns : 4 * 16 * ns; }
};

// Wave count and groups per load round of the SKINNY kernel for a partition of gpp groups.
struct SkinnyShape {
    int waves;  // waves per workgroup, each taking every waves-th group of the partition
    int gpw;    // groups whose loads one wave issues together
};

inline SkinnyShape skinny_shape(int mt, int gpp)
{
    const int max_waves = mt == 1 ? 16 : 8;
    const int max_gpw = mt == 4 ? 2 : 3;
    SkinnyShape sh;
    sh.waves = gpp < max_waves ? gpp : max_waves;
    const int per_wave = (gpp + sh.waves - 1) / sh.waves;
    sh.gpw = per_wave < max_gpw ? per_wave : max_gpw;
    return sh;
}

// Dense bf16 kernel: 2 x 2 waves, each 16*mt rows by 16*ns columns.
struct DenseTile {
    int mt;
    int ns;
    int block_m() const { return 2 * 16 * mt; }
    int block_n() const { return 2 * 16 * ns; }
};

hipError_t launch_w4a16(W4A16Tile tile, const void *A, const void *Wq, const void *scale,
                        const void *bias, void *out, int M, int N, int K, int s, bool vec_store,
                        hipStream_t stream);

hipError_t launch_w4a16_skinny(int mt, int gpw, int waves, const void *A, const void *Wq, const void *scale,
                               const void *bias, void *out, int M, int N, int K, int s, bool vec_store,
                               hipStream_t stream);

hipError_t launch_w4a16_wide(const void *A, const void *Wq, const void *scale, const void *bias, void *out,
                             int M, int N, int K, int s, bool vec_store, hipStream_t stream);

hipError_t launch_reduce(const void *partials, bool f32_partials, int s, size_t MN, void *C,
                         bool vec, hipStream_t stream);

hipError_t launch_dense(DenseTile tile, const void *A, const void *B, void *out, bool f32_out,
                        int M, int N, int K, int s, bool vec_store, hipStream_t stream);

}  // namespace qmm_impl
