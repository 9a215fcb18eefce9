// qmm_attn.hip -- split-KV decode attention with a log-sum-exp merge, for gfx950.
//
// skillsdirectory "Optimize Prefill vs Decode Kernels": decode attention splits the
// key/value sequence across workgroups, each computes a partial softmax over its key
// range, and a final pass merges the partials through their running maxima and sums
// (step 4, and the correctness notes: the partial max and sum of exponentials stay in
// fp32 and are combined with the online-softmax rule). The same split/reduce pattern
// as the split-K matmul, applied to the key axis.
//
// Operation (head dimension D = 128): for request b with len_b cached keys, query token
// i of Mq (the last Mq positions of the cache) and query head h, key/value head
// h / G (G = Hq / Hkv):
//     s_j = scale * Q[b,i,h,:] . K[b,h/G,j,:]  for j < len_b - Mq + 1 + i,
//     O[b,i,h,:] = sum_j softmax(s)_j V[b,h/G,j,:].
//
// Work decomposition: one workgroup per (request, key/value head, split p); split p
// covers keys [floor(p*len/S), floor((p+1)*len/S)). Its rows are the R = G*Mq queries
// that read that key/value head (row r = i*G + g), padded to RP = 4, 8 or 16 MFMA rows.
// The four waves take 64-key tiles round robin and keep their own running max m,
// running sum l and unnormalised accumulator (all fp32, scores in log2 units):
//   * scores: v_mfma_f32_16x16x32_bf16 with the keys as the first operand and the
//     queries as the second, straight from global memory (a lane loads 16 bytes of a
//     key row per 32-wide reduction step), so a lane holds four keys of one row;
//   * online softmax per tile: row max and row sum across the four lanes of a row
//     (two butterfly steps by lane swaps), rescale factor exp2(m_old - m_new);
//   * P . V on the vector ALU in fp32: the tile's probabilities go to LDS transposed
//     (key-major), a lane owns 8 head dimensions of every row for every fourth key of
//     the tile and streams the value rows with 16-byte loads;
//   * a tile's key and value loads are all issued before its first MFMA.
// The waves then merge in LDS (same rule), and the workgroup writes either O (one
// split) or its partial accumulator, max and sum; a second kernel merges the splits, 16
// at a time with the same rule.
// Masked and out-of-range keys read the split's last key (never past the cache) and
// get probability 0.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

constexpr int D = 128;       // head dimension
constexpr int TILE = 64;     // keys per wave tile
constexpr int NWAVE = 4;
constexpr float NEG_INF = -__builtin_inff();

struct AttnArgs {
    const uint16_t *Q, *K, *V;
    const int *lengths;
    uint16_t *O;
    float *part_acc;  // [S][rows][D]
    float *part_ml;   // [S][rows][2]: max (log2 units), sum
    int B, Mq, Hq, Hkv, Lmax, S;
    float scale_log2;  // softmax scale * log2(e)
};

// LDS: per wave the tile's probabilities, key-major [64][16], and the 16 rescale
// factors; reused for the cross-wave merge ([4][16][128] accumulators, [4][16] m, l).
struct AttnLds {
    union {
        struct {
            float p[NWAVE][TILE][16];
            float c[NWAVE][16];
        } t;
        struct {
            float acc[NWAVE][16][D];
            float m[NWAVE][16];
            float l[NWAVE][16];
        } mg;
    };
};

template <int RP>
__global__ void __launch_bounds__(64 * NWAVE)
attn_split_kernel(AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) AttnLds L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = a.S;
    const int p = blockIdx.x % S;
    const int bh = blockIdx.x / S;
    const int kvh = bh % a.Hkv;
    const int b = bh / a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int R = G * a.Mq;
    const int len = min(max(a.lengths[b], a.Mq), a.Lmax);
    // floor(p*len/S): in 32-bit unsigned arithmetic when (p+1)*len fits (len < 2^25, p < 64),
    // which keeps the software 64-bit division off the path from the length to the first
    // key address
    int k_lo, k_hi;
    if ((unsigned)len < (1u << 25)) {
        const unsigned lu = (unsigned)len, Su = (unsigned)S, pu = (unsigned)p;
        k_lo = (int)((pu * lu) / Su);
        k_hi = (int)(((pu + 1) * lu) / Su);
    } else {
        k_lo = (int)(((long long)p * len) / S);
        k_hi = (int)(((long long)(p + 1) * len) / S);
    }
    const size_t kv_base = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;

    // this lane's query row (scores) and its key limit
    const int qr = lane & 15;
    const int sl = lane >> 4;
    const int qi = qr / G;
    const int qlim = qr < R ? len - a.Mq + 1 + qi : 0;  // keys j < qlim are allowed
    bf16x8 qv[4];
    {
        const int h = kvh * G + (qr % G);
        const uint16_t *qrow = a.Q + (((size_t)b * a.Mq + (qr < R ? qi : 0)) * a.Hq + h) * D;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (qr < R) v = *reinterpret_cast<const uint4 *>(qrow + 32 * t + 8 * sl);
            qv[t] = as_bf16x8(v);
        }
    }

    // running state: m, l for row qr (replicated over the row's four lanes); the
    // accumulator of rows 0..RP-1 at head dimensions 8*(lane%16) .. +7, keys of subset lane/16
    float m_run = NEG_INF, l_run = 0.f;
    float acc[RP][8];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    const int dc = lane & 15;  // head-dimension chunk of the P.V part
    const int ku = lane >> 4;  // key subset of the P.V part

    for (int kt = k_lo + TILE * wave; kt < k_hi; kt += TILE * NWAVE) {
        // Every load of the tile is issued before the first use: the key rows of the
        // scores and the value rows of P.V (keys kt + ku + 4*jj) share one round trip.
        uint4 kv[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int key = min(kt + 16 * blk + qr, k_hi - 1);
            const uint16_t *krow = a.K + kv_base + (size_t)key * D;
#pragma unroll
            for (int t = 0; t < 4; ++t) kv[blk][t] = *reinterpret_cast<const uint4 *>(krow + 32 * t + 8 * sl);
        }
        uint4 vv[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int key = min(kt + ku + 4 * jj, k_hi - 1);
            vv[jj] = *reinterpret_cast<const uint4 *>(a.V + kv_base + (size_t)key * D + 8 * dc);
        }
        asm volatile("" ::: "memory");  // keep the loads above ahead of the arithmetic
        // scores of 4 blocks of 16 keys: lane holds keys kt + 16*blk + 4*sl + e of row qr
        f32x4 sc[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) d = mfma16x16x32(as_bf16x8(kv[blk][t]), qv[t], d);
            sc[blk] = d;
        }
        float tmax = NEG_INF;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kt + 16 * blk + 4 * sl + e;
                const float v = (key < k_hi && key < qlim) ? sc[blk][e] * a.scale_log2 : NEG_INF;
                sc[blk][e] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = xor32_max(xor16_max(tmax));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == NEG_INF ? 0.f : m_new;  // a row with no allowed key yet
        const float corr = exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = exp2f(sc[blk][e] - m_use);
                sc[blk][e] = pv;
                psum += pv;
            }
        psum = xor32_add(xor16_add(psum));
        l_run = l_run * corr + psum;
        m_run = m_new;
        // probabilities key-major, and each row's rescale factor, for the P.V part
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int e = 0; e < 4; ++e) L.t.p[wave][16 * blk + 4 * sl + e][qr] = sc[blk][e];
        if (sl == 0) L.t.c[wave][qr] = corr;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();

        float cr[RP];
#pragma unroll
        for (int r = 0; r < RP; r += 4) {
            const float4 c4 = *reinterpret_cast<const float4 *>(&L.t.c[wave][r]);
            cr[r] = c4.x; cr[r + 1] = c4.y; cr[r + 2] = c4.z; cr[r + 3] = c4.w;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= cr[r];
        // P.V: keys kt + ku + 4*jj of the tile
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int kl = ku + 4 * jj;  // key within the tile
            const uint32_t w[4] = {vv[jj].x, vv[jj].y, vv[jj].z, vv[jj].w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(w[e] << 16);
                v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
#pragma unroll
            for (int r = 0; r < RP; r += 4) {
                const float4 p4 = *reinterpret_cast<const float4 *>(&L.t.p[wave][kl][r]);
                const float pr[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r + rr][e] = __builtin_fmaf(pr[rr], v[e], acc[r + rr][e]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // the next tile rewrites this wave's LDS area
    }

    // sum the four key subsets (lanes dc, dc+16, dc+32, dc+48)
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[r][e];
            v = xor32_add(xor16_add(v));
            acc[r][e] = v;
        }
    __syncthreads();  // every wave is done with its tile area before the merge area is written
    if (ku == 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            *reinterpret_cast<float4 *>(&L.mg.acc[wave][r][8 * dc]) = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
            *reinterpret_cast<float4 *>(&L.mg.acc[wave][r][8 * dc + 4]) =
                make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
        }
    }
    if (sl == 0) {
        L.mg.m[wave][qr] = m_run;
        L.mg.l[wave][qr] = l_run;
    }
    __syncthreads();

    // merge the waves: thread t handles row r = t / 16 (r < RP), dims 8*(t%16) .. +7
    const int t = threadIdx.x;
    const int r = t >> 4;
    if (r < R) {
        const int dd = 8 * (t & 15);
        float m = NEG_INF;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) m = fmaxf(m, L.mg.m[w][r]);
        float lsum = 0.f;
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (m != NEG_INF) {
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                const float f = exp2f(L.mg.m[w][r] - m);
                lsum += f * L.mg.l[w][r];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += f * L.mg.acc[w][r][dd + e];
            }
        }
        const int i = r / G;
        const int h = kvh * G + r % G;
        const size_t row = ((size_t)b * a.Mq + i) * a.Hq + h;
        if (S == 1) {
            const float inv = 1.f / lsum;
            uint4 ov;
            ov.x = pack_bf16x2(o[0] * inv, o[1] * inv);
            ov.y = pack_bf16x2(o[2] * inv, o[3] * inv);
            ov.z = pack_bf16x2(o[4] * inv, o[5] * inv);
            ov.w = pack_bf16x2(o[6] * inv, o[7] * inv);
            *reinterpret_cast<uint4 *>(a.O + row * D + dd) = ov;
        } else {
            const size_t rows = (size_t)a.B * a.Mq * a.Hq;
            float *pa = a.part_acc + ((size_t)p * rows + row) * D + dd;
            *reinterpret_cast<float4 *>(pa) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4 *>(pa + 4) = make_float4(o[4], o[5], o[6], o[7]);
            if ((t & 15) == 0) {
                float *pm = a.part_ml + ((size_t)p * rows + row) * 2;
                pm[0] = m;
                pm[1] = lsum;
            }
        }
    }
}

// Merge of the S splits: one thread per (row, 8 head dimensions), splits in ascending order.
// One wave per workgroup: a single request has only 16 threads per query head (512 for 32
// heads), and 64-thread workgroups spread its partials' reads over four times as many CUs
// as 256-thread ones (single requests 3-6 % faster on MI355X).
__global__ void __launch_bounds__(64)
attn_merge_kernel(const float *__restrict__ part_acc, const float *__restrict__ part_ml, uint16_t *__restrict__ O,
                  int rows, int S)
{
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (size_t)rows * (D / 8)) return;
    const size_t row = t / (D / 8);
    const int dd = 8 * (int)(t % (D / 8));
    // The splits are read in batches of 16 whose loads are all issued before their use, so
    // up to 16 splits cost one memory round trip. Each batch is folded in with the online
    // rule: the running max m moves to the batch's max, the running sum and accumulator
    // are rescaled by exp2(m_old - m_new), and the batch's splits are added with weights
    // exp2(m_split - m_new). With one batch this is the plain two-pass merge (global max,
    // then the weighted sums). A split with no allowed key for this row stored max -inf,
    // sum 0 and a zero accumulator, so its weight is 0 and needs no branch.
    constexpr int BATCH = 16;
    float m = NEG_INF;
    float lsum = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < S; p0 += BATCH) {
        float2 ml[BATCH];
        float4 x[BATCH], y[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int p = min(p0 + u, S - 1);  // past S: re-read the last split, weight 0
            ml[u] = *reinterpret_cast<const float2 *>(part_ml + ((size_t)p * rows + row) * 2);
            const float *pa = part_acc + ((size_t)p * rows + row) * D + dd;
            x[u] = *reinterpret_cast<const float4 *>(pa);
            y[u] = *reinterpret_cast<const float4 *>(pa + 4);
        }
        float mb = NEG_INF;
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
            if (p0 + u < S) mb = fmaxf(mb, ml[u].x);
        const float m_new = fmaxf(m, mb);
        if (m_new == NEG_INF) continue;  // no allowed key in any split so far
        const float c = exp2f(m - m_new);  // 0 for the first batch with an allowed key
        lsum *= c;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= c;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float f = p0 + u < S ? exp2f(ml[u].x - m_new) : 0.f;
            lsum += f * ml[u].y;
            o[0] += f * x[u].x; o[1] += f * x[u].y; o[2] += f * x[u].z; o[3] += f * x[u].w;
            o[4] += f * y[u].x; o[5] += f * y[u].y; o[6] += f * y[u].z; o[7] += f * y[u].w;
        }
        m = m_new;
    }
    const float inv = 1.f / lsum;
    uint4 ov;
    ov.x = pack_bf16x2(o[0] * inv, o[1] * inv);
    ov.y = pack_bf16x2(o[2] * inv, o[3] * inv);
    ov.z = pack_bf16x2(o[4] * inv, o[5] * inv);
    ov.w = pack_bf16x2(o[6] * inv, o[7] * inv);
    *reinterpret_cast<uint4 *>(O + row * D + dd) = ov;
}

}  // namespace

namespace qmm_impl {

hipError_t launch_attn_decode(const void *Q, const void *K, const void *V, const int *lengths, void *O,
                              void *workspace, int B, int Mq, int Hq, int Hkv, int Lmax, float scale, int S,
                              hipStream_t stream)
{
    const int R = (Hq / Hkv) * Mq;
    if (R < 1 || R > 16 || S < 1) return hipErrorInvalidValue;
    const size_t rows = (size_t)B * Mq * Hq;
    AttnArgs a;
    a.Q = static_cast<const uint16_t *>(Q);
    a.K = static_cast<const uint16_t *>(K);
    a.V = static_cast<const uint16_t *>(V);
    a.lengths = lengths;
    a.O = static_cast<uint16_t *>(O);
    a.part_acc = static_cast<float *>(workspace);
    a.part_ml = S > 1 ? static_cast<float *>(workspace) + (size_t)S * rows * D : nullptr;
    a.B = B; a.Mq = Mq; a.Hq = Hq; a.Hkv = Hkv; a.Lmax = Lmax; a.S = S;
    a.scale_log2 = scale * 1.4426950408889634f;
    const dim3 grid((unsigned)((size_t)B * Hkv * S));
    (void)hipGetLastError();
    if (R <= 4)
        hipLaunchKernelGGL((attn_split_kernel<4>), grid, dim3(64 * NWAVE), 0, stream, a);
    else if (R <= 8)
        hipLaunchKernelGGL((attn_split_kernel<8>), grid, dim3(64 * NWAVE), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_split_kernel<16>), grid, dim3(64 * NWAVE), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    const size_t threads = rows * (D / 8);
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((threads + 63) / 64)), dim3(64), 0, stream,
                       a.part_acc, a.part_ml, a.O, (int)rows, S);
    return hipGetLastError();
}

}  // namespace qmm_impl
