/*
 * mxq -- scaled low-precision GEMM and routed fused-MoE experts for AMD MI355X (gfx950).
 *
 * C ABI of libmxq.so.  Conventions for every entry point:
 *
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never keeps them past the call and never allocates device memory.  Calls
 *    that need scratch take a caller-owned workspace (void* + size in bytes);
 *    the matching *_workspace_size() query returns the bytes needed.
 *  - Every call is asynchronous: it validates its arguments on the host,
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns.  Nothing synchronises with the host; launch grids are sized to
 *    upper bounds and surplus workgroups exit at once.
 *  - Scalars that live on the device (the per-tensor weight scale) are read by
 *    the kernels, so no host round trip is needed.
 *  - bf16 tensors are passed as 16-bit patterns, e4m3 as bytes (OCP FP8 E4M3FN,
 *    gfx950's native FP8: max 448, no infinities), e2m1 as packed nibbles (OCP
 *    MX FP4, element 2j in the low nibble of byte j), e8m0 as bytes (OCP MX
 *    scale, value 2^(e-127); 0xFF is not a valid scale).
 *  - Every pointer argument must be 16-byte aligned, and every row stride must
 *    keep rows 16-byte aligned, unless noted.
 *  - Return value: MXQ_OK or an error code (mxq_status_string() names it).  On
 *    an error nothing has been enqueued.
 *
 * Source pages cited below:
 *  [A] "vLLM PR 50949 review" -- routed FP8 / MXFP4 fused-MoE on CPU, with the
 *      BRGEMM-or-TinyGEMM choice taken per expert block from its real row
 *      count and column width (summary, implementation items 1-4, the
 *      moe_fp8.cpp and gemm.h listings).
 *  [B] "SGLang PR 32618 review" -- per-tensor FP8 W8A16 GEMM
 *      fp8_per_tensor_scaled_mm_cpu (implementation items 1-2, the fp8.py and
 *      test_gemm.py listings).
 *  [C] "SGLang PR 35605 review" -- block-wise FP8 W8A8 linear through
 *      scaled_mm (implementation items 1 and 3, the fp8_utils.py and
 *      test_xpu_fp8_linear.py listings).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mxq_status;

#define MXQ_OK 0
#define MXQ_ERR_NULL 1      /* a required pointer is NULL */
#define MXQ_ERR_SHAPE 2     /* sizes, strides or alignment not supported */
#define MXQ_ERR_BLOCK 3     /* block_size not in {[1,128], [128,128]} (page [C], fp8_utils.py listing) */
#define MXQ_ERR_DTYPE 4     /* unsupported dtype tag */
#define MXQ_ERR_WORKSPACE 5 /* workspace missing or too small */
#define MXQ_ERR_ARCH 6      /* the current device is not gfx950 */
#define MXQ_ERR_LAUNCH 7    /* a kernel launch failed (hipGetLastError) */
#define MXQ_ERR_ARG 8       /* any other invalid argument */
#define MXQ_ERR_SCRATCH 9   /* input larger than the static scratch of an allocation-free entry point */

/* dtype tags */
#define MXQ_DTYPE_BF16 0
#define MXQ_DTYPE_F32 1
#define MXQ_DTYPE_E4M3 2
#define MXQ_DTYPE_E2M1 3  /* packed OCP MX FP4, element 2j in the low nibble of byte j */

/* Text for a status code (static storage, never NULL). */
const char* mxq_status_string(mxq_status status);

/* ABI version of this header (bumped on any signature change or added entry point). */
int32_t mxq_abi_version(void);

/* Checks that `device` is a gfx950 GPU and makes it current.  Every other
 * entry point checks the current device on first use per device and returns
 * MXQ_ERR_ARCH on anything else (the GPU counterpart of the AMX-only assert of
 * page [B], fp8.py listing). */
mxq_status mxq_init(int32_t device);

/* ------------------------------------------------------------------ quantise
 * Per-token group quantisation to e4m3 (page [C], implementation item 1 and the
 * fp8_utils.py listing: activations get one fp32 scale per token per 128
 * columns, scale tensor [M, K/128]).  For each row and each group of 128
 * columns:  s = max(max|x|, 1e-10) / 448;  q = e4m3_rne(clamp(x / s, +-448))
 * with IEEE fp32 divisions; codes and scales are exact (bit-for-bit) results.
 *   x   bf16 [M, K], row stride ldx elements (ldx >= K, multiple of 8)
 *   q   e4m3 [M, K], contiguous (row stride K bytes)
 *   s   fp32 [M, K/128], contiguous
 *   group must be 128; K must be a multiple of 128 (else MXQ_ERR_BLOCK / MXQ_ERR_SHAPE).
 *   M == 0 or K == 0 is a no-op. */
mxq_status mxq_per_token_group_quant_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group,
                                         void* q, float* s, void* stream);

/* ------------------------------------------------------------------ per-tensor W8A16
 * out = bf16((A @ dec(W)^T) * scale + bias)   (page [B], implementation items 1-2
 * and the test_gemm.py listing; the per-tensor scale is the block scale with every
 * block equal, applied here once after the K loop).
 *   A      bf16 [M, K], row stride lda elements (lda >= K, multiple of 8)
 *   W      e4m3 [N, K], contiguous
 *   scale  fp32 device scalar (a 0-d or 1-element tensor)
 *   bias   NULL, or [N] of bias_dtype (MXQ_DTYPE_F32 or MXQ_DTYPE_BF16), added in fp32
 *   out    bf16 [M, N], row stride ldo elements (ldo >= N)
 *   workspace  mxq_fp8_scaled_mm_workspace_size(M, N, K) bytes (NULL allowed where it is 0),
 *          else MXQ_ERR_WORKSPACE: the fp32 partial sums of a K split (below).
 *   K must be a multiple of 32.  fp32 accumulation on the bf16 matrix cores.  Few rows (M <= 16,
 *   K >= 4096 a multiple of 128, at most 32 tiles of 16 x 128: ceil(N / 128) <= 32) run on the
 *   weight-streaming kernel: the scale multiplies each 128-wide K block's partial sum before it
 *   is added, and K may be cut into chunks whose partial sums are added in chunk order, so the
 *   sums are grouped differently from the tiles' (agreement within rounding; path and split
 *   depend on M, N and K only).  Otherwise, with K >= 6144, N a multiple of 8 and at most 128
 *   tiles, each tile's K range runs as 2, 4 or 8 chunks whose partial sums (each scaled) are
 *   added the same way (at most 16 MiB). */
size_t mxq_fp8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K);
mxq_status mxq_fp8_scaled_mm(const void* A, int64_t M, int64_t K, int64_t lda, const void* W, int64_t N,
                             const float* scale, const void* bias, int32_t bias_dtype, void* out, int64_t ldo,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ batched per-tensor W8A16
 * For z = 0 .. batch-1:  out[z] = bf16((A[z] @ dec(W[z])^T) * scale[z] + bias[z])  -- the batched
 * FP8 scaled GEMM that page [B] names as the existing use of its kernel (DeepSeek MLA's
 * per-head products, "Feature and motivation"); every entry is exactly the product
 * mxq_fp8_scaled_mm computes (same kernel, same arithmetic, bit-identical outputs).
 *   A      bf16, entry z = [M, K] at A + z * a_bstride elements, row stride lda elements
 *          (lda >= K, lda and a_bstride multiples of 8; 0 shares one A)
 *   W      e4m3, entry z = contiguous [N, K] at W + z * w_bstride bytes (w_bstride a
 *          multiple of 16; 0 shares one W)
 *   scale  fp32 device array, entry z at scale[z * scale_bstride] (0: one shared scale)
 *   bias   NULL, or bias_dtype (MXQ_DTYPE_F32 / MXQ_DTYPE_BF16), entry z = [N] at
 *          bias + z * bias_bstride elements (0: one shared bias)
 *   out    bf16, entry z = [M, N] at out + z * o_bstride elements, row stride ldo (>= N);
 *          entries may not overlap (o_bstride >= (M - 1) * ldo + N), else MXQ_ERR_SHAPE
 *   K must be a multiple of 32; 0 <= batch <= 65535 (batch, M or N == 0: no-op).  All
 *   buffers are the caller's device memory; the call enqueues on `stream` and returns. */
mxq_status mxq_fp8_scaled_bmm(const void* A, int64_t batch, int64_t M, int64_t K, int64_t lda, int64_t a_bstride,
                              const void* W, int64_t N, int64_t w_bstride, const float* scale,
                              int64_t scale_bstride, const void* bias, int32_t bias_dtype, int64_t bias_bstride,
                              void* out, int64_t ldo, int64_t o_bstride, void* stream);

/* ------------------------------------------------------------------ block-FP8 W8A8 linear
 * out[m, n] = bf16( sum_kb sa[m, kb] * sw[n / block_n, kb] * sum_{k in kb} dec(qa[m, k]) dec(W[n, k]) + bias[n] )
 * (page [C], implementation items 1 and 3 and the fp8_utils.py listing).
 *   A         a_dtype MXQ_DTYPE_BF16: bf16 [M, K] (row stride lda elements), quantised
 *             inside the call exactly as mxq_per_token_group_quant_fp8 does;
 *             a_dtype MXQ_DTYPE_E4M3: pre-quantised e4m3 [M, K] (row stride lda bytes)
 *             with a_scale fp32 [M, K/128] contiguous.  a_scale is ignored for bf16 input.
 *   W         e4m3 [N, K], contiguous
 *   w_scale   fp32 grid of logical shape [ceil(N / block_n), K / 128], element (i, j) at
 *             w_scale[i * ws_stride0 + j * ws_stride1] -- row-major and the transposed
 *             storage of page [C]'s load-time relayout both work, bit-identically.
 *   block_n, block_k   the weight block: (128, 128) or (1, 128); anything else -> MXQ_ERR_BLOCK
 *   bias      NULL or [N] of bias_dtype (fp32 or bf16)
 *   out       [M, N] of out_dtype, row stride ldo elements.  out_dtype must be
 *             MXQ_DTYPE_BF16 (page [C], fp8_utils.py listing: the output takes bf16 for
 *             pre-quantised input and the input's dtype otherwise, bf16 for every input
 *             this entry point accepts); anything else -> MXQ_ERR_DTYPE.
 *   workspace mxq_block_fp8_linear_workspace_size(M, N, K, a_dtype) bytes, or MXQ_ERR_WORKSPACE:
 *             bf16 input's quantised activations, and for the few-row cases below the fp32
 *             partial sums of a K split (at most 8 MiB); NULL allowed where the size is 0.
 *   K must be a multiple of 128.  FP8 matrix cores (16x16x128 per K block), fp32 accumulation.
 *   Few rows -- M <= 32 with K >= 4096, or M <= 64 where the row tiles would run at most 32
 *   workgroups, 96 for M <= 8 (ceil(M / t) * ceil(N / 128), t = 16, 32 or 64 rows for
 *   M <= 16, 32, 64) -- with
 *   N * K < 2^32 (and a tile's rows of its K chunk within the kernel's LDS) run on the
 *   weight-streaming kernel (tiles of 4 or 8 rows, each workgroup staging only its K chunk); that
 *   path may cut K into chunks of whole 128-wide blocks whose partial sums are added in chunk
 *   order, so its sums are grouped differently from the tiles' (the result agrees within
 *   rounding; path and split depend on M, N, K and the weight recipe only; the workspace size
 *   covers either recipe).  65..1024 rows on few 128 x 128 tiles
 *   with K >= 4096 (and M * K <= 8 M) split each tile's K range the same way (partial sums at
 *   most 16 MiB). */
size_t mxq_block_fp8_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t a_dtype);
mxq_status mxq_block_fp8_linear(const void* A, int32_t a_dtype, const float* a_scale, int64_t M, int64_t K,
                                int64_t lda, const void* W, int64_t N, const float* w_scale, int64_t ws_stride0,
                                int64_t ws_stride1, int32_t block_n, int32_t block_k, const void* bias,
                                int32_t bias_dtype, void* out, int32_t out_dtype, int64_t ldo, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ block-FP8 linear, no allocation
 * For callers that cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): mxq_block_fp8_linear with
 * the same arguments minus the workspace, same kernels and bit-identical results.  A bf16
 * input's quantised codes and scales go to a static device array of
 * MXQ_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it runs on until the
 * process ends, and so do the K-split partial sums of the few-row and few-tile paths; inputs
 * needing more than the array (mxq_block_fp8_linear_workspace_size bytes: M * K + 4 * M * K / 128
 * for bf16 input, i.e. about M * K <= 32.5 M, plus the partial sums -- at most 8 MiB for few
 * rows, 16 MiB for few tiles, whose M * K <= 8 M keeps the total within the array) return
 * MXQ_ERR_SCRATCH before anything is enqueued.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's array: calls that may overlap
 * on one GPU (different streams, no ordering between them) race and must not be issued; calls
 * on one stream are ordered and safe.  Nothing in the array needs to start at zero (the
 * quantiser and the split GEMM write all of it that is read).  e4m3 input uses the array only
 * for those partial sums. */
#define MXQ_NOALLOC_SCRATCH_BYTES (32u << 20)
mxq_status mxq_block_fp8_linear_noalloc(const void* A, int32_t a_dtype, const float* a_scale, int64_t M, int64_t K,
                                        int64_t lda, const void* W, int64_t N, const float* w_scale,
                                        int64_t ws_stride0, int64_t ws_stride1, int32_t block_n, int32_t block_k,
                                        const void* bias, int32_t bias_dtype, void* out, int32_t out_dtype,
                                        int64_t ldo, void* stream);

/* ------------------------------------------------------------------ MX-scaled quantise and linear
 * The MX block formats the pages name: MXFP4 expert weights (page [A], summary and
 * implementation item 2: e2m1 elements, one e8m0 scale per 32 elements of a row) and the
 * [1, 32] activation block recipe (page [C], implementation item 1), here as MXFP8: e4m3
 * elements with one e8m0 scale per 32 elements of a row.  The multiplications run on gfx950's
 * MX-scaled matrix instruction (V_MFMA_SCALE_F32_16X16X128_F8F6F4), which applies both
 * operands' e8m0 scales itself.
 *
 * mxq_mxfp8_quant: per row, per 32 columns (the OCP MX conversion rule):
 *   e = floor(log2(max|x|)) - 8 (8: the exponent of e4m3's largest normal), clamped to
 *   [-127, 127] (an all-zero block: -127);  s = e + 127 (e8m0);  q = e4m3_rne(clamp(x / 2^e, +-448)).
 *   Codes and scales are exact (bit-for-bit) results.
 *   x   bf16 [M, K], row stride ldx elements (ldx >= K, multiple of 8); K % 32 == 0
 *   q   e4m3 [M, K] contiguous;  s  e8m0 [M, K/32] contiguous.  M == 0 or K == 0: no-op.
 *
 * mxq_mx_linear: out[m, n] = bf16( sum_k a[m, k] w[n, k] + bias[n] ),
 *   a = dec(qa) * 2^(sa - 127), w = dec(qw) * 2^(sw - 127), fp32 accumulation.
 *   A        a_dtype MXQ_DTYPE_BF16: bf16 [M, K] (row stride lda elements), quantised inside
 *            the call exactly as mxq_mxfp8_quant does; a_dtype MXQ_DTYPE_E4M3: codes [M, K]
 *            (row stride lda bytes, a multiple of 16) with a_scale e8m0 [M, K/32] contiguous.
 *   workspace  mxq_mx_linear_workspace_size(M, N, K, a_dtype) bytes (NULL allowed where it is
 *            0), else MXQ_ERR_WORKSPACE: bf16 input's codes and scales, and -- with K >= 3072
 *            on at most 128 tiles (128 or 256 rows x 256 columns) -- the fp32 partial sums of
 *            a K split (2, 4 or 8 chunks added in chunk order: sums grouped differently,
 *            agreement within rounding; at most 16 MiB).
 *   W        w_dtype MXQ_DTYPE_E4M3: e4m3 [N, K];  MXQ_DTYPE_E2M1: packed e2m1 [N, K/2];
 *            contiguous, with w_scale e8m0 [N, K/32] contiguous (4-byte aligned).
 *   bias     NULL or [N] of bias_dtype (fp32 or bf16), added in fp32
 *   out      bf16 [M, N], row stride ldo elements
 *   K must be a multiple of 128; every operand below 4 GiB (else MXQ_ERR_SHAPE). */
mxq_status mxq_mxfp8_quant(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, void* s, void* stream);
size_t mxq_mx_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t a_dtype);
mxq_status mxq_mx_linear(const void* A, int32_t a_dtype, const void* a_scale, int64_t M, int64_t K, int64_t lda,
                         const void* W, int32_t w_dtype, int64_t N, const void* w_scale, const void* bias,
                         int32_t bias_dtype, void* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------------ expert sort / align
 * Groups the R = M * topk routed rows (flat id r = t * topk + k) by expert for the
 * block walk of page [A] (moe_fp8.cpp listing: expert_ids[mb], offsets[mb] with
 * m_size = offsets[mb+1] - offsets[mb], input token sorted_ids[mb * BLOCK_M + m] / topk).
 * Layout: experts ascending; inside an expert, flat ids ascending (stable); each
 * expert's rows cut into blocks of block_m (only its last block may be partial);
 * unused slots hold R; blocks past *num_blocks have expert -1 and offset R.
 *   topk_ids    int32 [M, topk]; ids outside [0, E) are ignored (those rows are dropped)
 *   sorted_ids  int32 [max_blocks * block_m]
 *   expert_ids  int32 [max_blocks]
 *   offsets     int32 [max_blocks + 1]
 *   num_blocks  int32 device scalar
 *   with max_blocks = mxq_moe_max_blocks(M, topk, E, block_m) = ceil(R / block_m) + min(E, R).
 *   1 <= E <= 512, 1 <= block_m <= 1024.  Runs as one workgroup; no host sync. */
int64_t mxq_moe_max_blocks(int64_t M, int32_t topk, int32_t E, int32_t block_m);
mxq_status mxq_moe_align(const int32_t* topk_ids, int64_t M, int32_t topk, int32_t E, int32_t block_m,
                         int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, int32_t* num_blocks,
                         void* stream);

/* ------------------------------------------------------------------ fused MoE experts
 * out[t] = bf16( sum_k topk_weights[t, k] * y[t*topk + k] ),
 *   y[r]  = ic1[r] @ w2[e]^T                                     (fp32)
 *   ic1   = bf16( silu(ic0[:, :I]) * ic0[:, I:] ),  silu(g) = g / (1 + exp(-g))
 *   ic0   = bf16( x[t] @ w1[e]^T + w1_bias[e] ),   e = topk_ids[t, k]
 * (page [A], implementation item 2 and the moe_fp8.cpp listing: stage 1 hidden @ w1
 * into a 2N-wide gate/up intermediate with an optional w1 bias, activation, stage 2
 * activation @ w2; the top-k combine weights each expert output by its routing
 * weight).  Rows [0, I) of w1 are the gate, rows [I, 2I) the up projection.
 * Each expert block picks its kernel from its own row count (page [A],
 * implementation items 1-2): a weight-streaming kernel for tiny blocks, MFMA
 * tiles of 16/32/64/128 rows otherwise (see mxq_moe_dispatch below; `dispatch`
 * NULL = per-block selection with the default bounds).
 *
 * mxq_fused_moe_fp8: block-FP8 weights.
 *   x            bf16 [M, H], contiguous
 *   topk_ids     int32 [M, topk];  topk_weights fp32 [M, topk]
 *   w1           e4m3 [E, 2I, H];  w1_scale fp32 [E, ceil(2I/128), H/128]
 *   w2           e4m3 [E, H, I];   w2_scale fp32 [E, ceil(H/128), I/128]
 *   w1_bias      NULL or fp32 [E, 2I]
 *   act_quant    0: W8A16 (bf16 activations into both stages);
 *                1: W8A8 (x and ic1 quantised per token per 128 columns, as
 *                   mxq_per_token_group_quant_fp8)
 *   weight_layout MXQ_LAYOUT_PLAIN: w1 / w2 as above;  MXQ_LAYOUT_TILED: w1 / w2 are
 *                the outputs of mxq_moe_prepack (the block scales keep their layout)
 *   out          bf16 [M, H], contiguous
 *   H and I must be multiples of 128.
 * mxq_fused_moe_mxfp4: MXFP4 weights, bf16 activations (W4A16).
 *   w1           packed e2m1 [E, 2I, H/2];  w1_scale e8m0 [E, 2I, H/32]
 *   w2           packed e2m1 [E, H, I/2];   w2_scale e8m0 [E, H, I/32]
 *   w1_bias      NULL or fp32 [E, 2I]
 *   weight_layout MXQ_LAYOUT_TILED: w1 / w2 from mxq_moe_prepack and w1_scale / w2_scale
 *                from mxq_moe_prepack_scales
 *   H and I must be multiples of 32.
 * Both: workspace of mxq_fused_moe_workspace_size(...) bytes (routing tables,
 * intermediates); experts that receive no rows are never read; 1 <= E <= 512.
 * The two layouts give bit-identical outputs.
 *
 * Per-call dispatch (`dispatch`, read during the call only; NULL = the defaults
 * {MXQ_DISPATCH_PER_BLOCK, 0, MXQ_TINY_ROWS_AUTO, MXQ_TINY_MFMA, MXQ_K_SPLIT_AUTO, MXQ_SORT_AUTO,
 * MXQ_FUSE_AUTO};
 * invalid fields -> MXQ_ERR_ARG):
 *   mode MXQ_DISPATCH_PER_BLOCK: each block's class from its own row count;
 *   mode MXQ_DISPATCH_FORCED: every block runs class `forced_class` (0 = tiny-block kernel,
 *        1 = 16-row, 2 = 32-row, 3 = 64-row, 4 = 128-row MFMA tiles) -- for tests;
 *   mode MXQ_DISPATCH_LAYER_AVERAGE: one class for the whole layer, chosen from
 *        max(1, M * topk / E) rows (the per-layer rule page [A] replaces; for
 *        ablation measurements).
 *   tiny_max_rows (0..16, or MXQ_TINY_ROWS_AUTO): largest block that takes the tiny-block
 *        class in per-block mode; AUTO = the measured crossover of the weight format: 4 rows
 *        for W8A8, 8 for W8A16, 4 for MXFP4; 0 = no tiny class.  With AUTO, bf16 activations,
 *        K <= 16384 and 16-byte aligned activation rows, a routing of more than AUTO x E rows
 *        has no tiny class: its tiny blocks take 16-row tiles in the tile launch.  When M <= 32 or
 *        M * topk <= 2 E the tiny class takes every block (taller ones in several passes);
 *        with bf16 activations, the MFMA tiny kernel, at most 4096 routed rows, E <= 512 and
 *        both stages' operands fitting the kernel's LDS budget, this case runs as two
 *        persistent expert-streaming kernels that group the routed rows by expert themselves
 *        (no sort and no block tables; the SiLU-and-mul ends stage 1) -- same arithmetic,
 *        bit-identical outputs.  Otherwise, for W8A8 with M * topk > 4096, K <= 16384 on both
 *        stages and operands below 4 GiB, every smaller class (the tiny one too, with the
 *        MFMA tiny kernel) folds into the 128-row class: its 128 x 256 tile keeps the GPU
 *        full with one launch per stage.  Column tiles: the 128 x 256 tile takes column
 *        tiles 256 wide; a last column tile of at most 128 columns takes the 128 x 128 tile.
 *   tiny_kernel: MXQ_TINY_MFMA (weights streamed into registers, K reduced by MFMAs, up
 *        to 8 rows per pass) or MXQ_TINY_GEMV (vector-ALU dot products with a wavefront
 *        reduction, 4 rows per pass; plain weight layout only -- with tiled weights the
 *        MFMA kernel runs).
 *   k_split (MXQ_K_SPLIT_AUTO, 1, 2, 4 or 8): with bf16 activations, at most 1024 routed
 *        rows, the MFMA tiny kernel and outside the expert-streaming case, a stage whose
 *        blocks give few tiles cuts each tile's K range into chunks (multiples of 256
 *        columns) that run as workgroups of their own and write fp32 partial sums to the
 *        workspace; the kernel after the stage sums them in chunk order.  AUTO: with at
 *        most 256 routed rows, the most chunks that keep min(E, M * topk) blocks of
 *        128-column tiles within 256 tiles (one per compute unit) -- except a stage of a
 *        routing the tiles can route themselves (see `sort`) whose largest grid of 16-, 32-
 *        or 64-row blocks fits 256 workgroups: it runs unsplit on those blocks; and a routing
 *        the expert-streaming kernels can take runs unsplit whatever `sort` and `fuse` say;
 *        1: never; 2 / 4 / 8: at most that many.  The workspace bounds the chunks to
 *        M * topk * chunks <= 2048.  Outputs agree with the unsplit call within rounding
 *        (the sums over K are grouped differently).
 *   sort MXQ_SORT_AUTO: small routings may skip the expert sort -- the expert-streaming case
 *        above, and, with bf16 activations, no tiny class, at most 2048 routed rows and
 *        E <= 512, when both stages run the direct-to-LDS 16/32/64/128-row tiles (K a
 *        multiple of 32 up to 16384, 16-byte aligned rows; plain MXFP4: K a multiple of 128),
 *        tiles that find their own rows from topk_ids (each expert's rows in the sort's
 *        order, cut into blocks of 16, 32 or 64); MXQ_SORT_ALWAYS: the sort kernel and its block
 *        tables always run.  Both give bit-identical outputs (every row's products are the
 *        same, whichever block holds it).
 *   fuse MXQ_FUSE_AUTO: with bf16 activations the SiLU-and-mul joins a neighbouring kernel
 *        where one fits -- the expert-streaming case above; the tiny-block kernel's stage-2
 *        row staging when the tiny class takes every block; and, when stage 1 runs wholly on
 *        the direct-to-LDS tiles (no tiny class) with whole K ranges and I a multiple of 64,
 *        the stage-1 epilogue: each tile pairs 64 gate rows of w1 with the matching 64 up rows
 *        and writes bf16(silu(g) * u) of its bf16-rounded outputs.  With top-1 routing, a
 *        self-routed stage 2 and whole K ranges, the top-k combine also joins the stage-2
 *        epilogue (out = bf16(weight * y), rows of dropped ids zeroed).  MXQ_FUSE_NONE:
 *        stage 1 always writes ic0, the standalone SiLU-and-mul forms ic1 and the combine
 *        kernel forms out.  Both give bit-identical outputs (the same rounding points, the
 *        same SiLU expression and the same combine arithmetic). */
#define MXQ_WEIGHTS_FP8_BLOCK 0
#define MXQ_WEIGHTS_MXFP4 1
#define MXQ_LAYOUT_PLAIN 0
#define MXQ_LAYOUT_TILED 1
#define MXQ_DISPATCH_PER_BLOCK 0
#define MXQ_DISPATCH_FORCED 1
#define MXQ_DISPATCH_LAYER_AVERAGE 2
#define MXQ_TINY_MFMA 0
#define MXQ_TINY_GEMV 1
#define MXQ_TINY_ROWS_AUTO (-1)
#define MXQ_K_SPLIT_AUTO 0
#define MXQ_SORT_AUTO 0
#define MXQ_SORT_ALWAYS 1
#define MXQ_FUSE_AUTO 0
#define MXQ_FUSE_NONE 1
typedef struct mxq_moe_dispatch {
  int32_t mode;
  int32_t forced_class;
  int32_t tiny_max_rows;
  int32_t tiny_kernel;
  int32_t k_split;
  int32_t sort;
  int32_t fuse;
} mxq_moe_dispatch;
size_t mxq_fused_moe_workspace_size(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                                    int32_t act_quant);
mxq_status mxq_fused_moe_fp8(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                             const int32_t* topk_ids, const float* topk_weights, const void* w1,
                             const float* w1_scale, const void* w2, const float* w2_scale, const float* w1_bias,
                             int32_t act_quant, int32_t weight_layout, const mxq_moe_dispatch* dispatch, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);
mxq_status mxq_fused_moe_mxfp4(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                               const int32_t* topk_ids, const float* topk_weights, const void* w1,
                               const void* w1_scale, const void* w2, const void* w2_scale, const float* w1_bias,
                               int32_t weight_layout, const mxq_moe_dispatch* dispatch, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Where the fused MoE keeps its intermediates inside the caller's workspace, so that a
 * caller (a test, a debugger) can read every stage of a call it made.  Fills
 * offsets[MXQ_MOE_WS_FIELDS] with byte offsets from the workspace base (-1 for a region
 * this configuration does not use) and returns MXQ_OK, or MXQ_ERR_SHAPE for sizes the
 * workspace query rejects.  After a call with act_quant = 1 (W8A8) the regions hold:
 *   SORTED_IDS / EXPERT_IDS / OFFSETS / NUM_BLOCKS  the align tables of mxq_moe_align for
 *        block_m = offsets[MXQ_MOE_WS_BLOCK_M] (the value, not an offset), without pad
 *        slots: only slots [offsets[mb], offsets[mb+1]) of block mb are meaningful
 *        (sorted_ids[mb * block_m + i] is the flat routed id of compact row offsets[mb] + i);
 *   QX / SX    x quantised as by mxq_per_token_group_quant_fp8 (e4m3 [M, H], fp32 [M, H/128]);
 *   IC0        bf16 [R, 2I]: stage-1 outputs (+ bias) by compact row;
 *   IC1_Q / IC1_S  e4m3 [R, I] + fp32 [R, I/128]: mxq_silu_and_mul of IC0, re-quantised;
 *   Y          fp32 [R, H]: stage-2 outputs by flat routed id t * topk + k;
 *   PARTIAL    fp32 K-split partial sums (bf16 activations only; -1 when M * topk > 1024).
 * With bf16 activations (act_quant = 0, and every MXFP4 call) the regions are scratch
 * whose contents depend on the kernels the dispatch picked (the expert-streaming path
 * writes neither the tables nor IC0). */
#define MXQ_MOE_WS_SORTED_IDS 0
#define MXQ_MOE_WS_EXPERT_IDS 1
#define MXQ_MOE_WS_OFFSETS 2
#define MXQ_MOE_WS_NUM_BLOCKS 3
#define MXQ_MOE_WS_QX 4
#define MXQ_MOE_WS_SX 5
#define MXQ_MOE_WS_IC0 6
#define MXQ_MOE_WS_IC1 7
#define MXQ_MOE_WS_IC1_Q 8
#define MXQ_MOE_WS_IC1_S 9
#define MXQ_MOE_WS_Y 10
#define MXQ_MOE_WS_BLOCK_M 11
#define MXQ_MOE_WS_PARTIAL 12
#define MXQ_MOE_WS_FIELDS 13
mxq_status mxq_fused_moe_workspace_layout(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                                          int32_t act_quant, int64_t* offsets);

/* The kernel plan a fused-MoE call of these sizes and this dispatch would run (host only: no
 * device is touched; the call's pointers are taken to be 16-byte aligned, as they must be).
 * Fills plan[MXQ_MOE_PLAN_FIELDS] and returns MXQ_OK; MXQ_ERR_SHAPE / MXQ_ERR_ARG for what the
 * call would refuse (M >= 1 here), MXQ_ERR_NULL for a NULL plan.  weights MXQ_WEIGHTS_*,
 * act_quant 0 / 1 (FP8 weights only), weight_layout MXQ_LAYOUT_*.  Fields:
 *   PATH      MXQ_MOE_PATH_SORTED (the sort kernel and its block tables, then the tile classes),
 *             MXQ_MOE_PATH_EXPERT_STREAM (every block tiny: two expert-streaming kernels, the
 *             other fields but SILU / COMBINE / K_SPLIT* zero or one), MXQ_MOE_PATH_SELF_ROUTED
 *             (the tiles find their own rows from topk_ids, no sort kernel);
 *   TILES     MXQ_MOE_TILES_RING (bf16 activations, direct-to-LDS tiles), _REGISTER (bf16
 *             activations, register-staged tiles), _W8A8, _W8A8_WIDE (W8A8 with the 128 x 256
 *             tile for its largest class);
 *   CLASSES   bit c set when block class c can occur (0 = tiny-block kernel, 1..4 = 16-, 32-,
 *             64-, 128-row tiles);
 *   BLOCK_M1 / BLOCK_M2  rows per routed block in stage 1 / 2 (128 on the sorted path);
 *   K_SPLIT1 / K_SPLIT2  K chunks per tile in stage 1 / 2;
 *   SILU      where the SiLU-and-mul runs: MXQ_MOE_SILU_KERNEL (its own kernel), _SPLIT_SUM (the
 *             kernel that also sums stage 1's K chunks), _STAGE1_EPILOGUE, _STAGE2_STAGING (the
 *             tiny-block kernel of stage 2), _EXPERT_STREAM;
 *   COMBINE   MXQ_MOE_COMBINE_KERNEL or _STAGE2_EPILOGUE (top-1, self-routed). */
#define MXQ_MOE_PLAN_PATH 0
#define MXQ_MOE_PLAN_TILES 1
#define MXQ_MOE_PLAN_CLASSES 2
#define MXQ_MOE_PLAN_BLOCK_M1 3
#define MXQ_MOE_PLAN_BLOCK_M2 4
#define MXQ_MOE_PLAN_K_SPLIT1 5
#define MXQ_MOE_PLAN_K_SPLIT2 6
#define MXQ_MOE_PLAN_SILU 7
#define MXQ_MOE_PLAN_COMBINE 8
#define MXQ_MOE_PLAN_FIELDS 9
#define MXQ_MOE_PATH_SORTED 0
#define MXQ_MOE_PATH_EXPERT_STREAM 1
#define MXQ_MOE_PATH_SELF_ROUTED 2
#define MXQ_MOE_TILES_RING 0
#define MXQ_MOE_TILES_REGISTER 1
#define MXQ_MOE_TILES_W8A8 2
#define MXQ_MOE_TILES_W8A8_WIDE 3
#define MXQ_MOE_SILU_KERNEL 0
#define MXQ_MOE_SILU_SPLIT_SUM 1
#define MXQ_MOE_SILU_STAGE1_EPILOGUE 2
#define MXQ_MOE_SILU_STAGE2_STAGING 3
#define MXQ_MOE_SILU_EXPERT_STREAM 4
#define MXQ_MOE_COMBINE_KERNEL 0
#define MXQ_MOE_COMBINE_STAGE2_EPILOGUE 1
mxq_status mxq_fused_moe_plan(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                              int32_t act_quant, int32_t weight_layout, const mxq_moe_dispatch* dispatch,
                              int32_t* plan);

/* ------------------------------------------------------------------ SiLU-and-mul
 * The activation between the two expert stages (page [A], implementation item 2 and the
 * moe_fp8.cpp listing: stage 1 writes a 2N-wide gate/up intermediate that the activation
 * reduces to N columns before stage 2):
 *   h[r, j] = bf16( silu(g) * u ),  g = ic0[r, j], u = ic0[r, I + j],  silu(g) = g / (1 + exp(-g)),
 * in fp32 on bf16 inputs.  q == NULL: h is written as bf16 [rows, I] to `out` (contiguous).
 * q != NULL: h is quantised per row per 128 columns exactly as
 * mxq_per_token_group_quant_fp8 quantises its input (codes e4m3 [rows, I] to q, scales
 * fp32 [rows, I/128] to s; `out` is not written and may be NULL) -- the W8A8 path's
 * re-quantisation of the stage-2 input.
 *   ic0  bf16 [rows, 2I], row stride ld_in elements (ld_in >= 2I, multiple of 8)
 *   I must be a multiple of 8 (of 128 when q != NULL).  rows == 0 is a no-op. */
mxq_status mxq_silu_and_mul(const void* ic0, int64_t rows, int64_t I, int64_t ld_in, void* out, void* q, float* s,
                            void* stream);

/* ------------------------------------------------------------------ load-time weight relayout
 * Converts routed-expert weights into the tiled layout the MoE kernels stream (page [B]:
 * the per-tensor GEMM takes prepacked or unpacked weights and its tests run both;
 * page [C]: layout work moved from the forward pass to weight loading).  Run once
 * when the weights are loaded; the caller owns both buffers.
 * mxq_moe_prepack: w [E, N, row_bytes] (e4m3 rows: row_bytes = K; packed e2m1: K/2)
 *   -> out of mxq_moe_prepack_size(E, N, row_bytes) bytes.  Rows are cut into
 *   16-row groups and 128-byte steps (the last step zero-padded); tile (e, g, s) is
 *   the 2048 bytes at ((e * N/16 + g) * S + s) * 2048, S = ceil(row_bytes / 128), and
 *   its byte 1024 h + 16 L holds bytes [32 (L / 16) + 16 h, +16) of row 16 g + L % 16
 *   (h in {0, 1}, L in [0, 64)).
 * mxq_moe_prepack_scales: e8m0 s [E, N, groups] -> out of
 *   mxq_moe_prepack_scales_size(E, N, groups) bytes; tile (e, g, s) is the 128 bytes at
 *   ((e * N/16 + g) * S + s) * 128, S = ceil(groups / 8), whose bytes 2 L and 2 L + 1
 *   hold groups 8 s + 2 (L / 16) and 8 s + 2 (L / 16) + 1 of row 16 g + L % 16 (0 past
 *   the row end).
 * N must be a multiple of 16 and row_bytes of 16 (else MXQ_ERR_SHAPE; the size queries
 * return 0); w and out 16-byte aligned. */
size_t mxq_moe_prepack_size(int64_t E, int64_t N, int64_t row_bytes);
size_t mxq_moe_prepack_scales_size(int64_t E, int64_t N, int64_t groups);
mxq_status mxq_moe_prepack(const void* w, int64_t E, int64_t N, int64_t row_bytes, void* out, void* stream);
mxq_status mxq_moe_prepack_scales(const void* s, int64_t E, int64_t N, int64_t groups, void* out, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
