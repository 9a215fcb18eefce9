/*
 * qmm.h -- C ABI of the split-K W4A16 group-128 quantized matmul for MI355X (gfx950).
 *
 * The library computes
 *
 *     C[M,N] = A[M,K] . dequant(W)[N,K]^T,   dequant(W)[n,k] = scale[n,k/128] * q[n,k] + bias[n,k/128]
 *
 * with bf16 activations A, 4-bit unsigned weights q packed eight per 32-bit word
 * along K, per-(row, 128-group) bf16 scale and bias, fp32 accumulation and a bf16
 * result (tiny-llm "Week 2 Day 7: Split-K Prefill": the W4A16 g128 kernel it
 * starts from, and the split of the reduction dimension it adds).
 *
 * When the unsplit output grid under-fills the GPU, an occupancy policy cuts the
 * reduction into s partitions on 128-value group boundaries (equal when s divides
 * the group count, as on the page; otherwise lengths that differ by one group); each
 * partition writes its own bf16 partial plane without atomics, and a second
 * kernel sums the planes in fp32 and casts once to bf16 (same page, Tasks 2-4).
 * When the grid is already full the policy returns s = 1 and the unsplit kernel
 * runs unchanged -- except for the large-M kernel under the MI355X preset, which
 * splits the columns of tiles left over after whole rounds of workgroup slots
 * (the split tail of qmm_splitk_plan, below). A dense bf16 split-K variant with fp32 partials is exported
 * beside it (gpu-kernels-explained "Split-K, streams and overlap", Concept).
 *
 * Layouts (all row-major, contiguous, no strides):
 *   A      bf16   [M][K]
 *   Wq     uint32 [N][K/8]   nibble i (bits 4i..4i+3) of word j holds q[n, 8j+i]
 *                            (qmm_wna16: [N][K*bits/32], 4- or 8-bit fields)
 *   scale  bf16   [N][K/128]   (qmm_wna16: [N][K/group_size])
 *   bias   bf16   [N][K/128]   (qmm_wna16: [N][K/group_size])
 *   C      bf16   [M][N]
 *   partials      [s][M][N]  bf16 (W4A16), fp32 (dense, and W4A16 through qmm_w4a16_g128_f32p)
 *   dense  A bf16 [M][K], B bf16 [N][K], C = A . B^T
 *
 * Ownership and execution: every pointer except those of qmm_splitk_plan is a
 * device pointer owned by the caller, including the workspace. The library
 * never allocates, frees or synchronises; it enqueues its kernels on `stream`
 * (a hipStream_t; NULL is the default stream) and returns. Results are defined
 * once the stream reaches that point. C must not overlap any input or the
 * workspace. Calls are thread-safe; the library holds no state, apart from the
 * static scratch array of qmm_w4a16_g128_noalloc.
 *
 * Errors: every entry point returns QMM_OK (0) or a negative QMM_ERR_* code.
 * All argument checks happen on the host before any launch, so a call that
 * returns an error has enqueued nothing and touched no memory. QMM_ERR_HIP
 * reports a launch failure from the HIP runtime.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QMM_OK = 0,
    QMM_ERR_ARG = -1,       /* NULL pointer, non-positive size, unknown dtype, group size != 128 */
    QMM_ERR_SHAPE = -2,     /* K not a multiple of 128 (32 for dense), split not allowed for the shape */
    QMM_ERR_ALIGN = -3,     /* A / Wq / B / workspace not 16-byte aligned, or an element misaligned */
    QMM_ERR_WORKSPACE = -4, /* split requested and workspace NULL or smaller than needed */
    QMM_ERR_HIP = -5,       /* a kernel launch failed (hipGetLastError) */
    QMM_ERR_SIZE = -6,      /* a size would overflow the library's 32-bit indexing (M*N, N*K, M*K > 2^37, or K >= 2^22) */
    QMM_ERR_SCRATCH = -7    /* qmm_w4a16_g128_noalloc: the split's planes exceed QMM_NOALLOC_SCRATCH_BYTES */
};

/* Partial-plane element types for qmm_splitk_reduce. */
enum { QMM_PARTIAL_BF16 = 0, QMM_PARTIAL_F32 = 1 };

/*
 * Occupancy policy (tiny-llm "Week 2 Day 7: Split-K Prefill", Task 3):
 *     base = ceil(M / tile_m) * ceil(N / tile_n)
 *     s    = min(cap, floor(target_blocks / base), floor(K / min_k_per_split), K/128)
 *     while s > 1 and (K/128) % s != 0: s -= 1
 *     s <= 1 -> the unsplit kernel
 * tile_m / tile_n = 0 mean "the block tile of the kernel this library launches
 * for that M" (the MI355X preset); the page's own rule counts 32 x 32 tiles.
 *
 * The small-M kernel runs M <= 64, and M <= 128 when N*K <= 2^24. Its tiles are 16*mt rows
 * (mt = 1, 2, 4 for M <= 16, 32, more) by 16 columns for M <= 32 with N*K <= 2^24 and for
 * M <= 8 with N <= 4096; else by 32
 * while 32-column tiles fit in 256 workgroups and K < 8192; else by 48 when 48-column tiles
 * fit in 256 workgroups, else by 64. With tile_m = tile_n = 0 and M <= 32, its partitions hold at least 2048 reduction
 * values (min_k_per_split is raised to 2048 in the rule): a shorter partition saves less
 * than the second pass costs; and the rule's last step (the divisor of K/128) is left out,
 * partition p covering groups [floor(p*G/s), floor((p+1)*G/s)). An unsplit grid of 16-column tiles with fewer tiles than 256
 * runs tiles of ceil(N / (256 / row blocks)) columns instead (block_n below), so that it
 * covers every CU once; the split rule still counts the 16-column tiles (tile_n). The large-M kernel runs the rest, with the tile of shortest
 * estimated critical path among 128 x 256 (two workgroups per CU up to M = 128), 256 x 256
 * (above M = 128) and 128 x 128 (only when its tiles are fewer than target_blocks, a pure
 * split at one workgroup per CU); ties go to the larger tiles. The estimate: rounds of
 * target_blocks workgroups times the 128 x 256 x 128 blocks each computes (a 256 x 256 tile
 * counts two, a 128 x 128 tile one half), plus half a block per partition of a split.
 * With tile_m = tile_n = 0 and the large-M kernel (T = base tiles, M-block
 * fastest, num_m tiles per column of tiles) the rule fills the kernel's workgroup
 * slots, target_blocks times the workgroups one CU holds (2 for its 128 x 256 tiles up to
 * M = 128, else 1),
 * with partitions that may differ by one group (no divisibility step); below,
 * target_blocks stands for that slot count:
 *     smax = min(cap, K/128, floor(K / min_k_per_split))
 *     T <  target_blocks: s = min(smax, floor(target_blocks / T)), every tile split
 *     T >= target_blocks: full = floor(T / target_blocks) * target_blocks, rounded down
 *         to a multiple of num_m, run unsplit; the tail T - full split in
 *         s = min(smax, floor(target_blocks / (T - full))) partitions
 *     s <= 1 -> the unsplit kernel
 * Partition p of a split tile covers groups [floor(p*G/s), floor((p+1)*G/s)), G = K/128.
 */
typedef struct qmm_policy {
    int tile_m;
    int tile_n;
    int target_blocks;
    int cap;
    int min_k_per_split;
} qmm_policy;

/* Result of qmm_splitk_plan. */
typedef struct qmm_plan {
    int s;                  /* chosen split count, >= 1; 1 = unsplit kernel, no workspace, no reduce */
    int base_tiles;         /* ceil(M/tile_m) * ceil(N/tile_n) under the policy's tile */
    int tile_m, tile_n;     /* tile the occupancy count used */
    int grid_x, grid_y, grid_z; /* grid of the matmul kernel this library launches for (M,N,K,s) */
    int block_m, block_n;   /* output tile of one workgroup of that kernel (block_n < tile_n for
                               a narrowed unsplit small-M grid) */
    size_t workspace_bytes; /* 2*s*M*N for s > 1, else 0 */
    int full_tiles;         /* kernel tiles computed unsplit ahead of the split ones: all of them
                               when s = 1, 0 for a uniform split, in between for a split tail */
} qmm_plan;

/* The page's rule: 32 x 32 tiles, 320 target blocks, cap 16, one group per partition. */
extern const qmm_policy QMM_POLICY_PAGE;
/* The rule re-tuned for MI355X (256 CUs): {0, 0, 256, 20, 512}, kernel tiles, 256 target
 * blocks (the CU count), cap 20, at least 512 K values per partition; used when s = 0 is
 * passed to qmm_w4a16_g128. */
extern const qmm_policy QMM_POLICY_MI355X;

/*
 * qmm_splitk_plan -- pick the split count for an (M, N, K) W4A16 g128 matmul.
 * Host only, pure: touches no device, allocates nothing.
 *   group_size must be 128. policy NULL selects QMM_POLICY_MI355X.
 *   Returns QMM_OK and fills *out, or QMM_ERR_ARG / QMM_ERR_SHAPE / QMM_ERR_SIZE.
 */
int qmm_splitk_plan(int M, int N, int K, int group_size, const qmm_policy *policy, qmm_plan *out);

/*
 * qmm_w4a16_g128 -- C = A . dequant(W)^T (tiny-llm "Week 2 Day 7", the public
 * matmul whose dispatcher picks the split and runs the partition and reduce kernels).
 *   s = 0  : the decomposition comes from qmm_splitk_plan(M, N, K, 128, NULL)
 *            (its s, and its full_tiles for the large-M kernel)
 *   s = 1  : the unsplit kernel (the control; also what the policy falls back to)
 *   s > 1  : explicit split of every tile into s partitions, 2 <= s <= K/128: partition p
 *            covers the 128-value groups [floor(p*G/s), floor((p+1)*G/s)), G = K/128
 *            (equal partitions when s divides G; otherwise they differ by one group).
 *            An explicit s equal to the plan's reproduces the plan's launch whenever the
 *            plan splits every tile (full_tiles = 0).
 *            Launches the split kernel, writing bf16 partial planes [s][M][N] into
 *            `workspace`, then the reduce into C (of the split tiles' columns only,
 *            when the plan runs the first tiles unsplit).
 *   workspace / workspace_bytes: needed only when the effective s > 1; at least
 *   2*s*M*N bytes, 16-byte aligned. May be NULL otherwise.
 *   Alignment: A and Wq 16-byte aligned; scale, bias and C 2-byte aligned.
 *   The effective s = 1 path is the same launch however it was reached, so its
 *   result is bitwise identical for s = 0 (when the policy picks 1) and s = 1.
 */
int qmm_w4a16_g128(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                   int M, int N, int K, int s, void *workspace, size_t workspace_bytes, void *stream);

/*
 * qmm_w4a16_g128_f32p -- qmm_w4a16_g128 with fp32 partial planes: each partition's
 * fp32 accumulator is stored unrounded and the reduce sums fp32 values, so the split
 * result differs from an fp32 sum over all of K only by summation order and the final
 * cast (tiny-llm "Week 2 Day 7: Split-K Prefill", Task 2 and Task 4: the partials may
 * be kept in FP32 at the cost of twice the workspace traffic).
 *   Same arguments, layouts, decomposition and errors as qmm_w4a16_g128, except that
 *   the workspace holds fp32 planes [s][M][N]: at least 4*s*M*N bytes when the
 *   effective s > 1. The effective s = 1 path is the same launch as qmm_w4a16_g128's,
 *   bitwise.
 */
int qmm_w4a16_g128_f32p(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                        int M, int N, int K, int s, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two passes of qmm_w4a16_g128 as separate calls (tiny-llm "Week 2 Day 7: Split-K
 * Prefill", Task 2 writes the partial planes, Task 4 sums them), for callers that run the
 * second pass themselves (on another stream, or fused into their own epilogue).
 *
 * qmm_w4a16_g128_pass1 -- the matmul launch of qmm_w4a16_g128 with the same arguments,
 * checks, errors and decomposition, and no second pass: every output tile computed over
 * the whole reduction is written to C; the partitions of split tiles go to the bf16
 * planes [s][M][N] in the workspace. *s_out receives the effective split and *n_lo_out
 * the first column whose outputs are still in the planes: those of columns [n_lo, N) of
 * every row (n_lo = N when s = 1; 0 when every tile is split; for the large-M kernel's
 * split tail, the first column of the tail tiles). Neither output pointer may be NULL;
 * both are host pointers, written before the call returns.
 *
 * qmm_splitk_reduce_cols -- the second pass over columns [n_lo, N): for every row m and
 * n_lo <= n < N, C[m][n] = bf16_rne(sum over p = 0..s-1, in this order, in fp32, of
 * partials[p][m][n]); the other columns of C are not touched. partials as for
 * qmm_splitk_reduce; 0 <= n_lo < N.
 *
 * qmm_w4a16_g128_pass1, then qmm_splitk_reduce_cols(workspace, QMM_PARTIAL_BF16, s, M, N,
 * n_lo, C) when s > 1, leaves C bitwise equal to qmm_w4a16_g128's result.
 */
int qmm_w4a16_g128_pass1(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                         int M, int N, int K, int s, void *workspace, size_t workspace_bytes,
                         int *s_out, int *n_lo_out, void *stream);

int qmm_splitk_reduce_cols(const void *partials, int partial_dtype, int s, int M, int N, int n_lo,
                           void *C, void *stream);

/*
 * qmm_w4a16_g128_noalloc -- qmm_w4a16_g128 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * bf16 partial planes of a split live in a static device array of the library, of
 * QMM_NOALLOC_SCRATCH_BYTES (64 MiB), instead of a caller's workspace. The caller still
 * passes the inputs and C.
 *   Same arguments (without the workspace), layouts, decomposition, kernels, results and
 *   errors as qmm_w4a16_g128; the result is bitwise equal to qmm_w4a16_g128's for the same
 *   arguments. A split whose planes (2*s*M*N bytes for the effective s > 1) would exceed the
 *   array returns QMM_ERR_SCRATCH and launches nothing (every Qwen3-4B projection up to
 *   M = 128, and q, k, v, o and down at M = 2048, fit under the plan; gate and up at M = 2048
 *   need 199 MB: pass s = 1 there).
 *   The first call on a device looks up that device's copy of the array (with the device
 *   current; `stream` must belong to the current device); no call allocates, frees or
 *   synchronises. Each GPU's array is held until the process ends and is shared by every
 *   call on that GPU: calls that overlap in time on one GPU (on different streams or
 *   threads) race on it and must be serialised by the caller. Nothing in it needs to start
 *   at zero; it keeps the last call's planes.
 */
#define QMM_NOALLOC_SCRATCH_BYTES (64u << 20)
int qmm_w4a16_g128_noalloc(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                           int M, int N, int K, int s, void *stream);

/*
 * Other weight-only formats (skillsdirectory "Optimize Prefill vs Decode Kernels",
 * step 6: weight-only W4A16 and W8A16 with the dequantisation fused into the matmul
 * loop), on the same kernels, plan and reduce as qmm_w4a16_g128.
 *
 *   bits        4 or 8: unsigned codes q in [0, 2^bits), packed 32/bits per 32-bit word
 *               along K, lowest field first: field i (bits bits*i .. bits*i+bits-1) of word
 *               j of row n holds q[n, (32/bits)*j + i]. Wq is uint32 [N][K*bits/32].
 *   group_size  32, 64 or 128: scale and bias are bf16 [N][K/group_size], and
 *               w[n,k] = scale[n, k/group_size] * q[n,k] + bias[n, k/group_size].
 *   K must be a multiple of 128. The split partitions K into blocks of 128 values (each a
 *   whole number of groups): s = 0 asks qmm_wna16_plan, 1 <= s <= K/128 splits as for
 *   qmm_w4a16_g128 (partition p covers blocks [floor(p*G/s), floor((p+1)*G/s)), G = K/128).
 *   partial_dtype QMM_PARTIAL_BF16 (workspace >= 2*s*M*N bytes) or QMM_PARTIAL_F32
 *   (>= 4*s*M*N bytes) when the effective s > 1.
 *   qmm_wna16(4, 128, QMM_PARTIAL_BF16, ...) is qmm_w4a16_g128, launch for launch, and
 *   qmm_wna16(4, 128, QMM_PARTIAL_F32, ...) is qmm_w4a16_g128_f32p.
 *   Errors as qmm_w4a16_g128; an unsupported bits, group_size or partial_dtype is
 *   QMM_ERR_ARG.
 */
int qmm_wna16(int bits, int group_size, int partial_dtype, const void *A, const void *Wq,
              const void *scale, const void *bias, void *C, int M, int N, int K, int s,
              void *workspace, size_t workspace_bytes, void *stream);

/* qmm_splitk_plan for a (bits, group_size) format: the same rule, with the large-M
 * kernel's workgroups per CU for that format's LDS footprint. workspace_bytes is the
 * bf16-partial size. Host only, pure. QMM_ERR_ARG for an unsupported format. */
int qmm_wna16_plan(int bits, int group_size, int M, int N, int K, const qmm_policy *policy,
                   qmm_plan *out);

/*
 * qmm_w4a16_g128_streamk -- the same product with the stream-K decomposition of the
 * large-M kernel (the persistent-style decomposition that gives every workgroup an equal
 * share of multiply-adds across tile boundaries; the split of the pages' Task 2 with
 * unequal, tile-crossing partitions): the (tile, 128-value block) units, tile-major, are
 * cut into `workgroups` near-equal contiguous ranges. A tile one workgroup covers whole
 * is written to C directly (bitwise the unsplit kernel's result); the pieces of a shared
 * tile go to per-workgroup slots of the workspace as bf16 and a fix-up kernel adds them in
 * reduction order in fp32, with one cast to bf16. Deterministic, no atomics.
 *   M > 64 (QMM_ERR_SHAPE otherwise: small M runs another kernel).
 *   workgroups = 0: one per workgroup slot of the GPU (256 times the workgroups one CU
 *   holds for this shape's tile), at most units / 4 (four blocks, 512 reduction values, per
 *   workgroup, the MI355X preset's floor) and at least 1; else 1 .. units, where
 *   units = ceil(M/BM) * ceil(N/256) * K/128 and BM = 128 for M <= 128, else 256.
 *   workspace >= qmm_streamk_workspace_bytes(M, N, K, workgroups), 16-byte aligned.
 *   Other arguments, layouts and errors as qmm_w4a16_g128.
 */
int qmm_w4a16_g128_streamk(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                           int M, int N, int K, int workgroups, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Workspace of qmm_w4a16_g128_streamk: 2 * P * BM * 256 * 2 bytes for its P workgroups;
 * 0 for shapes it does not take. Host only. */
size_t qmm_streamk_workspace_bytes(int M, int N, int K, int workgroups);

/*
 * qmm_w4a16_gemv -- the same product for decode-sized M (1 to 8 rows) on a matrix-vector
 * kernel with no matrix-core padding (tiny-llm "Week 2 Day 7", Benchmark Analysis:
 * decode runs on a separate matvec). Every packed weight is read once per call. On the
 * Qwen3-4B projections on MI355X it is faster than qmm_w4a16_g128 at M = 1 (down 6.5 against
 * 8.1 us); from M = 4 on, the matmul's 16-row MFMA tile is faster (the dot-product work
 * here grows with M). A workgroup computes 16 output columns, or 10 for one or two rows
 * when that spreads the columns over more CUs.
 *   M in 1..8, else QMM_ERR_SHAPE. Same layouts, alignment, ownership and errors as
 *   qmm_w4a16_g128.
 *   s = 0  : qmm_gemv_min_split(M, K), the smallest split whose partitions fit the
 *            kernel's staging of A in LDS;
 *   s >= 1 : explicit; must divide K/128 and K/s must fit (QMM_ERR_SHAPE otherwise):
 *            K/s <= 10240, m8*K/s <= 30720 and, for m8 = 8, K/s <= 4096, where m8 is M
 *            rounded up to 1, 2, 4 or 8.
 *   s > 1 writes bf16 planes [s][M][N] into `workspace` (at least 2*s*M*N bytes,
 *   16-byte aligned) and merges them with the reduce of qmm_splitk_reduce.
 */
int qmm_w4a16_gemv(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                   int M, int N, int K, int s, void *workspace, size_t workspace_bytes, void *stream);

/* The split qmm_w4a16_gemv uses for s = 0 (>= 1), or QMM_ERR_ARG / QMM_ERR_SHAPE /
 * QMM_ERR_SIZE. Host only. */
int qmm_gemv_min_split(int M, int K);

/*
 * qmm_splitk_reduce -- C[i] = bf16_rne( sum over p = 0..s-1, in this order, in fp32,
 * of partials[p][i] ) for i < M*N (tiny-llm "Week 2 Day 7", Task 4: one output
 * element per thread, FP32 sum, one cast to the model dtype).
 *   partial_dtype: QMM_PARTIAL_BF16 or QMM_PARTIAL_F32. partials holds s planes of
 *   M*N elements back to back, aligned to its element size. s >= 1.
 */
int qmm_splitk_reduce(const void *partials, int partial_dtype, int s, int M, int N, void *C,
                      void *stream);

/*
 * qmm_bf16_splitk -- dense C = A . B^T with bf16 A[M][K], B[N][K], fp32 accumulation
 * (gpu-kernels-explained "Split-K, streams and overlap", Concept: a small output
 * with a long k cut into s slices, partial sums added by a second pass).
 *   K must be a multiple of 32. The reduction is cut into s near-equal partitions of
 *   units of 64 values when K is a multiple of 64, else of 32-value granules: partition p
 *   covers units [floor(p*U/s), floor((p+1)*U/s)), U = K/64 (K/32), so any 1 <= s <= U
 *   is allowed (QMM_ERR_SHAPE beyond). Bounds on the 64-value grid keep every row's reads
 *   on whole 128-byte lines.
 *   s = 0 picks s with the MI355X occupancy rule over this kernel's tile.
 *   s = 1 writes C directly; s > 1 writes fp32 partial planes [s][M][N] to the
 *   workspace (>= 4*s*M*N bytes, 16-byte aligned), then reduces them into C.
 *   A and B 16-byte aligned; C 2-byte aligned.
 */
int qmm_bf16_splitk(const void *A, const void *B, void *C, int M, int N, int K, int s,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * qmm_attn_decode -- split-KV decode attention with a log-sum-exp merge (skillsdirectory
 * "Optimize Prefill vs Decode Kernels", step 4 and its correctness notes: the key/value
 * sequence is split across workgroups, each keeps an fp32 running max and sum of
 * exponentials, and a final pass merges the partial results with the online-softmax rule).
 *
 *   For request b (lengths[b] cached keys), query token i < Mq (the last Mq positions of
 *   the cache) and query head h < Hq, with key/value head h / (Hq/Hkv):
 *     s_j = scale * Q[b,i,h,:] . K[b,h/G,j,:]   for j < lengths[b] - Mq + 1 + i
 *     O[b,i,h,:] = sum_j softmax(s)_j * V[b,h/G,j,:]
 *   Layouts (bf16, row-major, contiguous): Q and O [B][Mq][Hq][head_dim], K and V
 *   [B][Hkv][Lmax][head_dim]; lengths: device int32 [B], each in [Mq, Lmax] (values
 *   outside are clamped into that range on the device).
 *   head_dim must be 128, Hq a multiple of Hkv and (Hq/Hkv)*Mq <= 16 (QMM_ERR_SHAPE).
 *   s = 0: qmm_attn_decode_split(B, Hkv, Lmax); s >= 1 (at most 64): split p of request b
 *   covers keys [floor(p*len/s), floor((p+1)*len/s)). s > 1 needs a workspace of
 *   qmm_attn_decode_workspace_bytes(B, Mq, Hq, s) bytes, 16-byte aligned (fp32 partial
 *   accumulators, maxima and sums), and launches the merge after the split kernel.
 *   Q, K, V and O 16-byte aligned, lengths 4-byte aligned. Errors as qmm_w4a16_g128;
 *   a non-finite scale is QMM_ERR_ARG.
 */
int qmm_attn_decode(const void *Q, const void *K, const void *V, const int *lengths, void *O,
                    int B, int Mq, int Hq, int Hkv, int Lmax, int head_dim, float scale, int s,
                    void *workspace, size_t workspace_bytes, void *stream);

/* The split qmm_attn_decode uses for s = 0: enough workgroups for one per CU
 * (ceil(256 / (B*Hkv))), at most Lmax/64 (a 64-key tile per split), at most
 * max(16, Lmax/512) (past the 16 splits the merge reads in one round trip, only with 512
 * keys per split) and 32, at least 1 (fitted to split sweeps of the Qwen3-4B decode shapes
 * on MI355X). Host only; QMM_ERR_ARG for a non-positive size. */
int qmm_attn_decode_split(int B, int Hkv, int Lmax);

/* Workspace bytes of qmm_attn_decode for split s: s*B*Mq*Hq*(128 + 2)*4, 0 for s <= 1. */
size_t qmm_attn_decode_workspace_bytes(int B, int Mq, int Hq, int s);

/* Human-readable name of a status code (static storage, never NULL). */
const char *qmm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
