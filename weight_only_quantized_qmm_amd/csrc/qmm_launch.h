// qmm_launch.h -- internal interface between the C-ABI host code (qmm_api.cpp)
// and the gfx950 kernels (*.hip). Not installed; the public ABI is include/qmm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace qmm_impl {

// Output tile handled by one workgroup of the W4A16 kernel: 4 waves side by side
// along N, each owning 16*ns columns and all 16*mt rows of the block.
struct W4A16Tile {
    int mt;  // 16-row MFMA subtiles per block (1, 2, 4, 8)
    int ns;  // 16-column MFMA subtiles per wave (1, 2, 4)
    int block_m() const { return 16 * mt; }
    int block_n() const { return 4 * 16 * ns; }
};

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

hipError_t launch_reduce(const void *partials, bool f32_partials, int s, size_t MN, void *C,
                         bool vec, hipStream_t stream);

hipError_t launch_dense(DenseTile tile, const void *A, const void *B, void *out, bool f32_out,
                        int M, int N, int K, int s, bool vec_store, hipStream_t stream);

}  // namespace qmm_impl
