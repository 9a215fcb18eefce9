// qmm_reduce.hip -- the split-K merge pass for gfx950.
//
// C[i] = bf16( ((P[0][i] + P[1][i]) + ...) + P[s-1][i] ), every addition in fp32,
// one round-to-nearest-even cast at the end (tiny-llm "Week 2 Day 7: Split-K
// Prefill", Task 4: one output element per thread, FP32 sum of all partitions,
// a single cast to the model dtype). The planes are s contiguous arrays of
// M*N elements; the sum runs in ascending partition order so that the result
// is reproducible bit for bit.
//
// MI355X layout: the op is a pure stream (reads s*M*N partial elements, writes
// M*N outputs), so each lane owns eight consecutive outputs and moves them with
// 128-bit loads and stores (one 16-byte load per bf16 plane, two per fp32 plane),
// up to eight planes' loads in flight at once.
// The scalar variant handles element counts or pointers that are not 16-byte
// multiples, one output per lane.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

// Raw bits of eight consecutive partial elements: one 16-byte load of bf16, two of fp32.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    uint4 x;
    __device__ __forceinline__ void load(const uint16_t *p) { x = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <>
struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ float get(int e) const {
        const float4 &v = e < 4 ? a : b;
        const int k = e & 3;
        return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    }
};

__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float *p) { return *p; }

// Planes whose loads a lane has in flight together: every load of a chunk is issued
// before the first addition, so a lane waits for one memory round trip per chunk
// instead of one per plane (a loop that adds each plane as it arrives makes s
// dependent trips, which at M = 128 left the merge at a third of HBM bandwidth).
constexpr int kChunk = 8;

// acc[0..7] = sum over p < s of plane p's eight elements at offset off, ascending p.
template <typename T>
__device__ __forceinline__ void sum8(const T *__restrict__ part, size_t MN, size_t off, int s, float acc[8])
{
    for (int p0 = 0; p0 < s; p0 += kChunk) {
        Raw8<T> r[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k)
            if (p0 + k < s) r[k].load(part + (size_t)(p0 + k) * MN + off);
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            if (p0 + k >= s) break;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = (p0 + k == 0) ? r[k].get(e) : acc[e] + r[k].get(e);
        }
    }
}

template <typename T>
__device__ __forceinline__ float sum1(const T *__restrict__ part, size_t MN, size_t off, int s)
{
    float acc = 0.f;
    for (int p0 = 0; p0 < s; p0 += kChunk) {
        float v[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k)
            if (p0 + k < s) v[k] = load1(part + (size_t)(p0 + k) * MN + off);
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            if (p0 + k >= s) break;
            acc = (p0 + k == 0) ? v[k] : acc + v[k];
        }
    }
    return acc;
}

__device__ __forceinline__ uint4 pack8(const float acc[8])
{
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    return o;
}

template <typename T>
__global__ void __launch_bounds__(256)
reduce_vec8(const T *__restrict__ part, uint16_t *__restrict__ C, int s, size_t MN)
{
    const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= MN) return;  // MN is a multiple of 8 on this path
    float acc[8];
    sum8(part, MN, i, s, acc);
    *reinterpret_cast<uint4 *>(C + i) = pack8(acc);
}

template <typename T>
__global__ void __launch_bounds__(256)
reduce_scalar(const T *__restrict__ part, uint16_t *__restrict__ C, int s, size_t MN)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    C[i] = (uint16_t)f32_to_bf16(sum1(part, MN, i, s));
}

// Columns [n_lo, N) of planes [s][M][N]: W = N - n_lo columns per row; eight
// consecutive columns per lane when W, N and n_lo are multiples of 8, else one.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256)
reduce_cols(const T *__restrict__ part, uint16_t *__restrict__ C, int s, int M, int N, int n_lo)
{
    const int W = N - n_lo;
    const int per = VEC ? 8 : 1;
    const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * per;
    if (i >= (size_t)M * (size_t)W) return;
    const int m = (int)(i / (size_t)W);
    const int n = n_lo + (int)(i % (size_t)W);
    const size_t off = (size_t)m * (size_t)N + n;
    const size_t MN = (size_t)M * (size_t)N;
    if (VEC) {
        float acc[8];
        sum8(part, MN, off, s, acc);
        *reinterpret_cast<uint4 *>(C + off) = pack8(acc);
    } else {
        C[off] = (uint16_t)f32_to_bf16(sum1(part, MN, off, s));
    }
}

template <typename T>
hipError_t launch_t(const T *part, int s, size_t MN, uint16_t *C, bool vec, hipStream_t stream)
{
    const size_t per_thread = vec ? 8 : 1;
    const size_t threads = (MN + per_thread - 1) / per_thread;
    const dim3 grid((unsigned)((threads + 255) / 256));
    (void)hipGetLastError();
    if (vec)
        hipLaunchKernelGGL((reduce_vec8<T>), grid, dim3(256), 0, stream, part, C, s, MN);
    else
        hipLaunchKernelGGL((reduce_scalar<T>), grid, dim3(256), 0, stream, part, C, s, MN);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

hipError_t launch_reduce(const void *partials, bool f32_partials, int s, size_t MN, void *C,
                         bool vec, hipStream_t stream)
{
    if (f32_partials)
        return launch_t(static_cast<const float *>(partials), s, MN, static_cast<uint16_t *>(C), vec, stream);
    return launch_t(static_cast<const uint16_t *>(partials), s, MN, static_cast<uint16_t *>(C), vec, stream);
}

template <typename T>
hipError_t launch_cols_t(const T *p, int s, int M, int N, int n_lo, uint16_t *c, bool vec, hipStream_t stream)
{
    const size_t elems = (size_t)M * (size_t)(N - n_lo);
    const size_t per_thread = vec ? 8 : 1;
    const size_t threads = (elems + per_thread - 1) / per_thread;
    const dim3 grid((unsigned)((threads + 255) / 256));
    (void)hipGetLastError();
    if (vec)
        hipLaunchKernelGGL((reduce_cols<T, true>), grid, dim3(256), 0, stream, p, c, s, M, N, n_lo);
    else
        hipLaunchKernelGGL((reduce_cols<T, false>), grid, dim3(256), 0, stream, p, c, s, M, N, n_lo);
    return hipGetLastError();
}

hipError_t launch_reduce_cols(const void *partials, bool f32_partials, int s, int M, int N, int n_lo, void *C,
                              bool vec, hipStream_t stream)
{
    if (n_lo < 0 || n_lo >= N) return hipErrorInvalidValue;
    uint16_t *c = static_cast<uint16_t *>(C);
    if (f32_partials) return launch_cols_t(static_cast<const float *>(partials), s, M, N, n_lo, c, vec, stream);
    return launch_cols_t(static_cast<const uint16_t *>(partials), s, M, N, n_lo, c, vec, stream);
}

}  // namespace qmm_impl
