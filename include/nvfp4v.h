/* nvfp4v: NVFP4 skinny verify-GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation. A speculative-decoding verify pass applies every linear layer
 * of the target model to all rows of a draft tree in one forward pass; the
 * weights are stored with four bits per weight and one scale per 16 weights,
 * so the pass is a skinny GEMM that streams 4-bit weights from HBM and whose
 * cost is flat in the row count until a tile boundary is crossed
 * (TandemLLM manual, "What TandemLLM is", 1.2 "Two levers"; StairCut research
 * page, "What it says"). This library computes, for M = 1..128 rows (up to
 * four sequences' trees of 32 rows checked in one pass: TandemLLM manual, 1.4
 * "What runs today", requests decoding together share one verify pass),
 *
 *     C[M, N] (fp32) = ts * A[M, K] (bf16) * W[N, K]^T,
 *     W[j, k] = E2M1(code[j, k]) * E4M3(scale[j, k / 16])
 *
 * Reading of the format (the pages give only "4 bits, one scale per 16"):
 * E2M1 codes (sign, 2-bit exponent with bias 1, 1 mantissa bit: magnitudes
 * 0, .5, 1, 1.5, 2, 3, 4, 6), an OCP E4M3 ("FN": bias 7, no infinities,
 * 0x7F/0xFF are NaN) scale for every 16 consecutive elements along K, and an
 * fp32 tensor scale ts.
 *
 * Canonical (interchange) format, row-major, caller-owned:
 *     codes  uint8 [N][K/2]   byte b of row j holds k = 2b (low nibble) and
 *                             k = 2b + 1 (high nibble)
 *     scales uint8 [N][K/16]  E4M3 byte of block k/16
 * Packed (device) format: an opaque byte permutation of the canonical bytes,
 * zero-padded to N % 16 == 0 and K % 128 == 0, produced by nvfp4v_pack() and
 * consumed by nvfp4v_verify_gemm(); its size is nvfp4v_packed_bytes(). When
 * N % 16 == 0 and K % 128 == 0 it is exactly N*K/2 + N*K/16 bytes.
 *
 * Conventions for every call:
 *   - "dev" pointers are device memory on the context's GPU, "host" pointers
 *     are host memory. The caller owns every buffer it passes in.
 *   - Sizes are element counts (int64_t), never bytes unless named *_bytes.
 *   - Return 0 on success or a negative NVFP4V_E_* status. All argument checks
 *     run on the host before any HIP call; on error nothing is launched and
 *     no output is written. No C++ exception crosses this interface.
 *   - Calls that take a hipStream_t enqueue work and return without
 *     synchronising; faults during execution surface at the caller's next
 *     synchronisation. Launch failures return NVFP4V_E_HIP and the hipError_t
 *     is kept (nvfp4v_last_hip_error).
 *   - Calls that share one context must not run concurrently (they share the
 *     context's split-K workspace); enqueue them on one stream.
 *   - The K-reduction order is fixed for a given (N, K, M, device): repeated
 *     calls return bitwise identical C (TandemLLM manual, 1.7 "The paper":
 *     the 4-bit kernels keep a fixed reduction order).
 */
#ifndef NVFP4V_H
#define NVFP4V_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4V_OK 0
#define NVFP4V_E_INVALID_ARG (-1) /* null pointer / null context / bad enum   */
#define NVFP4V_E_SHAPE (-2)       /* K % 16 != 0, N < 1, K < 16, too large     */
#define NVFP4V_E_M_RANGE (-3)     /* M < 1 or M > NVFP4V_MAX_M                  */
#define NVFP4V_E_ALIGN (-4)       /* a device pointer is not 16-byte aligned   */
#define NVFP4V_E_HIP (-5)         /* a HIP runtime or launch error             */
#define NVFP4V_E_FAULT (-6)       /* injected by NVFP4V_FAULT=launch (testing) */
#define NVFP4V_E_NONFINITE (-7)   /* quantiser input holds NaN or Inf          */
#define NVFP4V_E_WORKSPACE (-8)   /* the request exceeds the context workspace */
#define NVFP4V_E_TIMEOUT (-9)     /* a persistent pass gave up at a grid barrier */
#define NVFP4V_E_DISPATCH (-10)   /* split-K pieces of a row block ran on two XCDs */
#define NVFP4V_E_TABLE (-11)      /* a tile-table file is unreadable or malformed  */

#define NVFP4V_MAX_M 128

typedef struct nvfp4v_ctx nvfp4v_ctx;

/* Create a context on HIP device `device` (>= 0). It holds the device's
 * properties, the tile table, and a split-K workspace (partial sums and
 * arrival counters) allocated here once, so that nvfp4v_verify_gemm never
 * allocates and can be captured in a HIP graph. The caller destroys it.
 * tile_table_path: NULL for the built-in gfx950 table (the library's
 * tables/gfx950.txt, compiled in), else a table file in that format, whose
 * rules are tried before the built-in ones (see nvfp4v_load_tile_table;
 * TandemLLM manual, "What TandemLLM is", 1.1 "The test environment": the
 * kernels' tile tables come from the board they run on).
 * Create also runs a short synchronous dispatch probe: when the device deals
 * the work-groups of a launch out to its XCDs round-robin by linear id (as
 * gfx950 does in its one-partition mode), split-K GEMMs exchange their
 * partial sums through the L2 of the one XCD that runs a row block's pieces;
 * otherwise, or with NVFP4V_SPLITK_EXCHANGE=memory in the environment,
 * through memory. Both give bitwise identical C. */
int nvfp4v_create(nvfp4v_ctx **out, int device, const char *tile_table_path);
void nvfp4v_destroy(nvfp4v_ctx *ctx);

/* (Re)load the context's tile table from a text file; NULL returns it to the
 * built-in table alone. Format: lines of whitespace-separated fields, '#'
 * starts a comment; one "arch gfx950" line (the only arch this library is built
 * for), then rules
 *     rule <nrt_lo> <nrt_hi> <nkt_lo> <nkt_hi> <m_lo> <m_hi> <kernel> <R> <ksplit>
 * (at most 64): a GEMM of nrt row tiles (16 weight rows each) and nkt k-tiles
 * (256 elements of K each) at M rows takes the plan of the first rule whose
 * inclusive ranges hold all three ("*" is an open end); kernel "reg" (waves
 * split K, R row tiles per work-group: 1, 2, 4 or 8) or "lds" (activations
 * staged in LDS, waves split N, R row tiles per wave: 1, or 2 up to 32 rows);
 * ksplit work-groups along K (1..64), summed in a fixed order. GEMMs that no
 * rule holds take the built-in table. Host only (no HIP call); the loaded rules
 * apply to the context's later calls. NVFP4V_PLAN=r=<R>,ks=<S> (or
 * n:r=<R>,ks=<S> for the LDS variant) in the environment still overrides both.
 * Errors: INVALID_ARG, TABLE (unreadable file, unknown field, wrong arch, a
 * range, R or ksplit out of bounds, a kernel not built for some M of its
 * range, more than 64 rules); on error the previous table stays. */
int nvfp4v_load_tile_table(nvfp4v_ctx *ctx, const char *path);

/* Synchronise the device, then report the device-side errors that GEMMs on
 * this context recorded since it was created or last reported one:
 * NVFP4V_E_DISPATCH if the pieces of some split-K row block ran on different
 * XCDs, so that their exchange through one XCD's L2 could not meet (the C of
 * that call is undefined; the context then clears the record and its arrival
 * counters and exchanges through memory from then on), else NVFP4V_OK.
 * Errors: INVALID_ARG, HIP. */
int nvfp4v_device_status(nvfp4v_ctx *ctx);

/* Synchronise the device, then write to *units_host the number of GEMM work
 * units on this context that met a marker in the fp16 copy of their packed
 * activations and were computed again from the bf16 copy (see
 * nvfp4v_act_packed_bytes), counted since the context was created or last
 * reported NVFP4V_E_DISPATCH. A measurement: with O(1) activations only values
 * below 2^-25 in magnitude cause it. Errors: INVALID_ARG, HIP. */
int nvfp4v_f16_redone(nvfp4v_ctx *ctx, uint64_t *units_host);

/* Size in bytes of the opaque context object. Host-only tests use it to build a
 * zeroed stand-in context whose every argument check runs on the host and
 * returns before any HIP call (an all-zero context has an empty workspace). */
size_t nvfp4v_ctx_size(void);

/* Human-readable text for a status code (static storage). */
const char *nvfp4v_strerror(int status);
/* The hipError_t behind the last NVFP4V_E_HIP on this context (0 if none). */
int nvfp4v_last_hip_error(const nvfp4v_ctx *ctx);

/* ---- Format ------------------------------------------------------------ */

/* Quantise fp32 host weights w[N][K] to the canonical format (host buffers
 * codes[N][K/2], scales[N][K/16]). Per 16-element block along K:
 *     s = E4M3_RNE(absmax / 6)    (fp64, round to nearest even, saturating
 *                                   at 448; may be 0)
 *     code = s == 0 ? +0 : E2M1_RNE(w / s)   (fp64, ties to the even mantissa,
 *                                   saturating at 6, sign kept so tiny
 *                                   negatives become -0)
 * The pages say only that the weights were quantised onto the NVFP4 grid
 * ("Installing TandemLLM", 3.12); this absmax/6 rule is the plain reading.
 * Errors: INVALID_ARG, SHAPE (K % 16, N < 1), NONFINITE. */
int nvfp4v_quantize_host(const float *w_host, int64_t n, int64_t k, uint8_t *codes_host,
                         uint8_t *scales_host);

/* The same quantiser on the GPU: w_dev fp32 [N][K] -> codes_dev [N][K/2],
 * scales_dev [N][K/16], byte-identical to nvfp4v_quantize_host. Non-finite
 * weights are not reported on this path (the bytes are then unspecified);
 * check inputs on the host if they can hold NaN/Inf. */
int nvfp4v_quantize(nvfp4v_ctx *ctx, const float *w_dev, int64_t n, int64_t k,
                    uint8_t *codes_dev, uint8_t *scales_dev, hipStream_t stream);

/* Round fp32 host values to E4M3 bytes (nearest even, saturating at +-448,
 * NaN rejected with NONFINITE). Used to store scale values given directly. */
int nvfp4v_encode_e4m3_host(const float *x_host, int64_t count, uint8_t *out_host);

/* Bytes of the packed (device) format for an N x K matrix. 0 for bad shapes. */
size_t nvfp4v_packed_bytes(int64_t n, int64_t k);

/* Canonical (device buffers) -> packed (device buffer of nvfp4v_packed_bytes).
 * Padding bytes are written as zero codes with zero scales.
 * Errors: INVALID_ARG, SHAPE, ALIGN (packed_dev), HIP. */
int nvfp4v_pack(nvfp4v_ctx *ctx, const uint8_t *codes_dev, const uint8_t *scales_dev, int64_t n,
                int64_t k, void *packed_dev, hipStream_t stream);

/* Packed -> canonical (inverse of nvfp4v_pack). */
int nvfp4v_unpack(nvfp4v_ctx *ctx, const void *packed_dev, int64_t n, int64_t k,
                  uint8_t *codes_dev, uint8_t *scales_dev, hipStream_t stream);

/* ---- The verify GEMM ---------------------------------------------------- */

/* C[M][N] = ts * A[M][K] * W[N][K]^T.
 *   a_dev      bf16 bit patterns, row-major [M][K] (row stride K), 16-byte
 *              aligned, K % 8 == 0 for that alignment to hold per row
 *   packed_dev nvfp4v_pack output for the N x K weights, 16-byte aligned
 *   c_dev      fp32, row-major [M][N], 16-byte aligned; fully overwritten
 * M in 1..128. Does not allocate; safe to capture in a HIP graph. A is packed
 * into the context's 16 MiB buffer (all M rows at once when they fit, else
 * one block of 64 rows at a time; K up to 65536, else WORKSPACE), then the
 * GEMM runs over it. For M > 64, where the tile table names the wide unit,
 * one launch covers all rows; otherwise one launch per block of 64 rows, in
 * turn.
 * Errors: INVALID_ARG, SHAPE, M_RANGE, ALIGN, WORKSPACE, HIP, FAULT. */
int nvfp4v_verify_gemm(nvfp4v_ctx *ctx, const uint16_t *a_dev, int64_t m, int64_t k,
                       const void *packed_dev, int64_t n, float ts, float *c_dev,
                       hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): nvfp4v_verify_gemm without a
 * context, on the current HIP device. It allocates nothing: its scratch (the
 * packed activations of one block of 64 rows, split-K partial sums and arrival
 * counters) is one file-scope device array of 24 MiB + 64 KiB that every GPU
 * the library runs on holds until the process ends. Limits: K such that a
 * block of 64 rows of packed activations (both copies) fits 16 MiB
 * (K <= 65536), and plans whose split-K partials fit 8 MiB and use at most
 * 4096 row blocks, else WORKSPACE. It uses the built-in tile table and
 * exchanges split-K partials through memory, one launch per block of 64 rows;
 * C equals nvfp4v_verify_gemm's bitwise wherever that also runs one launch per
 * block (always up to 64 rows; above, shapes the tile table gives the wide
 * unit sum in another order and agree to the same tolerance). Every call on a GPU
 * shares that GPU's array (a small kernel clears its counters at the start of
 * each call): calls that overlap on one GPU (other streams, other threads)
 * race and must not be made. Errors: INVALID_ARG, SHAPE, M_RANGE, ALIGN,
 * WORKSPACE, HIP, FAULT. */
int nvfp4v_verify_gemm_static(const uint16_t *a_dev, int64_t m, int64_t k, const void *packed_dev,
                              int64_t n, float ts, float *c_dev, hipStream_t stream);

/* ---- Tree-verify attention ------------------------------------------------
 * One attention layer of the verify pass for the M rows of one draft tree
 * (row 0 the root token, then the tree's nodes, parents before children)
 * against the committed context (the served model mixes Gated DeltaNet layers
 * with attention layers: TandemLLM manual, "What TandemLLM is", 1.1 "The test
 * environment"; every row of the tree goes through each layer in one pass:
 * 1.2 "Two levers"; the cost is measured per context length from 1k to 32k:
 * release post, the paragraph on what checking 8 to 32 guesses costs):
 *     O[i][h] = sum_j softmax_j(scale * q[i][h] . k[j][h / G]) v[j][h / G]
 * over the positions j row i sees: every context position 0..T-1 and the tree
 * rows on its own path to the root, itself included, whose keys and values
 * are at cache positions T + row. G = Hq / Hkv query heads share a key/value
 * head. bf16 inputs, fp32 arithmetic (the softmax weights enter the value
 * product as two bf16 terms), fp32 output; bitwise reproducible.
 *
 * Caches (device, caller-owned, nvfp4v_kv_cache_bytes(cap, Hkv, D) bytes each):
 * an opaque MFMA-fragment order of keys and values for positions 0..cap-1
 * (cap a multiple of 32), written by nvfp4v_kv_write. Head dim D = 128. */
#define NVFP4V_ATTN_HEAD_DIM 128
#define NVFP4V_ATTN_MAX_ROWS 32 /* G * M <= 32 query columns per key/value head */
size_t nvfp4v_kv_cache_bytes(int64_t cap, int hkv, int d); /* 0 for a bad shape */

/* Write n rows of keys and values, bf16 [n][Hkv][D] row-major each, to cache
 * positions pos0 .. pos0 + n - 1 (a device kernel on `stream`; does not
 * allocate or synchronise). Errors: INVALID_ARG, SHAPE (D != 128, Hkv not in
 * 1..64, cap not a positive multiple of 32, positions beyond cap), ALIGN, HIP,
 * FAULT. */
int nvfp4v_kv_write(nvfp4v_ctx *ctx, const uint16_t *k_rows_dev, const uint16_t *v_rows_dev, int64_t n,
                    int64_t pos0, int hkv, int d, int64_t cap, uint16_t *k_cache_dev,
                    uint16_t *v_cache_dev, hipStream_t stream);

/* Workspace of nvfp4v_tree_attention (0 for a bad shape). Its first 1024 bytes
 * are arrival tickets that must be zero before the first call (hipMemset once);
 * every call leaves them zero. */
size_t nvfp4v_tree_attention_workspace_bytes(int64_t ctx_len, int64_t m, int hq, int hkv, int d);

/* Enqueue the attention of M tree rows (1 <= M, (Hq / Hkv) * M <= 32) on
 * `stream`. q: bf16 [M][Hq][D]; k_cache / v_cache: positions 0..ctx_len-1 the
 * context, ctx_len + i tree row i (ctx_len + M <= cap); parent_rows: HOST
 * array of M int32, parent_rows[0] = -1, 0 <= parent_rows[i] < i; scale: the
 * score scale (1/sqrt(D) for plain attention); o: fp32 [M][Hq][D]. The keys
 * and values of positions beyond ctx_len + M are never used (any bits there,
 * NaN included, leave O unchanged). Work: one work-group per (key/value head,
 * chunk of positions), the last of a head merging the chunks in order. Does
 * not allocate or synchronise; calls sharing a workspace must not overlap.
 * Errors: INVALID_ARG (null pointer, bad parent_rows, non-finite scale),
 * SHAPE, M_RANGE, ALIGN, WORKSPACE, HIP, FAULT. */
int nvfp4v_tree_attention(nvfp4v_ctx *ctx, const uint16_t *q_dev, const uint16_t *k_cache_dev,
                          const uint16_t *v_cache_dev, int64_t cap, int64_t ctx_len, int64_t m, int hq,
                          int hkv, int d, const int32_t *parent_rows, float scale, float *o_dev,
                          void *ws_dev, size_t ws_bytes, hipStream_t stream);

/* The chunking nvfp4v_tree_attention uses for a shape on the context's GPU
 * (chunks per key/value head: one work-group per CU, where more than 16 query
 * columns over a context of up to 8192 positions take one work-group per
 * 16-column block, and longer contexts with more than 16 columns every
 * work-group slot once chunks exceed 2048 positions; at least 352 positions
 * and at most 64 chunks; positions per chunk), for reports.
 * Errors: INVALID_ARG, SHAPE, M_RANGE, HIP. */
int nvfp4v_tree_attention_plan(nvfp4v_ctx *ctx, int64_t ctx_len, int64_t m, int hq, int hkv, int d,
                               int *nchunks, int *chunk);

/* Activations pre-packed in the GEMM's MFMA fragment order, for callers that
 * produce the next GEMM's input themselves (the chained pass writes them from
 * its glue kernels). nvfp4v_verify_gemm does this packing internally, into the
 * context's buffer, before each call. More than 64 rows are packed as
 * consecutive blocks of 64 rows (the last one shorter), each in the layout of
 * its own row count. The packed form holds A twice in that order: the bf16
 * values, then (half the packed size further on) each value times 2^8 as fp16
 * where that conversion is exact (0, or magnitudes in [2^-25, 2^8)) and a NaN
 * marker elsewhere. The GEMM computes from the fp16 copy, whose products with
 * the dequantised weights are exact (an fp16 dequantisation costs one VALU
 * operation per weight, the bf16 one two), and computes any work unit whose
 * sums meet a marker again from the bf16 copy: C is the same, bitwise, as
 * computed from the bf16 values alone (NVFP4V_F16=0 in the environment does
 * that for every unit).
 *   nvfp4v_act_packed_bytes: bytes of the packed form of A[M][K], both
 *     copies (0 if bad).
 *   nvfp4v_pack_activations: a_dev bf16 [M][K] row-major -> act_dev (16-byte
 *     aligned, nvfp4v_act_packed_bytes bytes). Errors: INVALID_ARG, M_RANGE,
 *     SHAPE, ALIGN, HIP, FAULT.
 *   nvfp4v_verify_gemm_pa: as nvfp4v_verify_gemm (the same launches for
 *     M > 64), with A given packed. */
size_t nvfp4v_act_packed_bytes(int64_t m, int64_t k);
int nvfp4v_pack_activations(nvfp4v_ctx *ctx, const uint16_t *a_dev, int64_t m, int64_t k,
                            void *act_dev, hipStream_t stream);
int nvfp4v_verify_gemm_pa(nvfp4v_ctx *ctx, const void *act_dev, int64_t m, int64_t k,
                          const void *packed_dev, int64_t n, float ts, float *c_dev,
                          hipStream_t stream);

/* ---- The FP8 output head ------------------------------------------------ */

/* The output head applied after the last layer of a verify pass: the served
 * model keeps it in FP8 (TandemLLM manual, "What TandemLLM is", 1.2 "Two
 * levers"). The pages give neither the FP8 variant nor the scale granularity;
 * read here as OCP E4M3 ("FN") codes with one fp32 scale per weight row:
 *   s(j) = fp32(absmax_k |w(j,k)| / 448), code = E4M3_RNE(w / s) saturating at
 *   448 with the sign kept (every code +0 when s(j) == 0).
 *   nvfp4v_fp8_packed_bytes: bytes of the packed head for N x K (0 if N < 1,
 *     K < 16, K % 16 != 0, N > 2^28 or K > 2^22).
 *   nvfp4v_fp8_quantize_host: fp32 w[N][K] (host) -> codes u8[N][K] row-major
 *     and row_scales fp32[N] (host, caller-owned). Errors: INVALID_ARG, SHAPE,
 *     NONFINITE (NaN or Inf in w).
 *   nvfp4v_fp8_pack_host: codes + row scales (host) -> the packed layout in a
 *     caller-owned host buffer of nvfp4v_fp8_packed_bytes bytes (copy it to the
 *     device once; offline). Errors: INVALID_ARG, SHAPE.
 *   nvfp4v_fp8_head_gemm: C[M][N] fp32 = A[M][K] * (s . W8)^T for bf16 A
 *     (device, row-major, 16-byte aligned), the packed head (device, 16-byte
 *     aligned), C (device, row-major, 16-byte aligned, fully overwritten).
 *     M in 1..128, one launch per block of 64 rows (each block of A is packed
 *     into the context's buffer first). Does not allocate. Errors:
 *     INVALID_ARG, M_RANGE, SHAPE, ALIGN, WORKSPACE, HIP, FAULT.
 *   nvfp4v_fp8_head_gemm_pa: the same with A given packed
 *     (nvfp4v_pack_activations). */
size_t nvfp4v_fp8_packed_bytes(int64_t n, int64_t k);
int nvfp4v_fp8_quantize_host(const float *w_host, int64_t n, int64_t k, uint8_t *codes_host,
                             float *row_scales_host);
int nvfp4v_fp8_pack_host(const uint8_t *codes_host, const float *row_scales_host, int64_t n,
                         int64_t k, void *packed_host);
int nvfp4v_fp8_head_gemm(nvfp4v_ctx *ctx, const uint16_t *a_dev, int64_t m, int64_t k,
                         const void *packed_dev, int64_t n, float *c_dev, hipStream_t stream);
int nvfp4v_fp8_head_gemm_pa(nvfp4v_ctx *ctx, const void *act_dev, int64_t m, int64_t k,
                            const void *packed_dev, int64_t n, float *c_dev, hipStream_t stream);

/* The kernel variant and tiling the tile table picks for (N, K, M): writes a
 * short description into buf (NUL-terminated, truncated to len). */
int nvfp4v_describe_plan(nvfp4v_ctx *ctx, int64_t n, int64_t k, int64_t m, char *buf, size_t len);

/* ---- Staircase sweep ---------------------------------------------------- */

/* Measure the verify GEMM's duration for every M in [m_lo, m_hi] on an N x K
 * weight matrix (the per-M cost "staircase" that StairCut prices; StairCut
 * research page, "What it says"). The call allocates its own buffers:
 * max(1, ceil(rotate_bytes / packed)) weight copies filled with valid random
 * codes and scales, cycled so timing does not hit a cache-resident copy; it
 * runs `warmup` untimed launches, then five batches of `reps` back-to-back
 * launches, each batch between one pair of HIP events on an internal stream,
 * and writes the median batch's time per launch in microseconds to
 * us_out[M - m_lo] (a pair of events around one launch would add a launch's
 * dispatch latency). The activations are packed once per M (as the chained
 * pass does), so the timed launches are the GEMM kernel alone (M > 64: one
 * launch per block of 64 rows, counted together). Synchronous. */
int nvfp4v_staircase(nvfp4v_ctx *ctx, int64_t n, int64_t k, int m_lo, int m_hi, int warmup,
                     int reps, size_t rotate_bytes, double *us_out);


/* ---- StairCut: cutting a draft tree on the measured staircase ----------- */

/* The cut rule of the pages' router (StairCut research page, "What it says":
 * each round is priced on the measured verify-cost staircase and keeps the tree
 * size that pays the most expected tokens per millisecond; release post: the
 * candidate tree is cut to the node count with the most expected committed
 * tokens per millisecond at the measured price, snapping to 7, 15, 23 or 31
 * nodes). Host code; no GPU is touched.
 *   us_by_rows  host double[max_rows]: us_by_rows[r - 1] is the measured time
 *               in microseconds of a verify pass over r rows (the staircase).
 *   parent      host int32[n_nodes]: the draft tree, nodes in an order where a
 *               parent precedes its children; -1 = a child of the root (the
 *               last committed token).
 *   p_accept    host double[n_nodes] in [0, 1]: probability that the model's
 *               own token at the node's position is the node's token, given
 *               that its parent was accepted. Siblings are different tokens at
 *               one position, so the probabilities of a node's children sum to
 *               at most 1.
 *   sizes       host int32[n_sizes] candidate node counts (NULL: 7, 15, 23,
 *               31); a candidate above n_nodes means the whole tree.
 * A cut to n nodes keeps the n nodes with the highest path probability P (the
 * product of p along the root path; those nodes always form a subtree), is
 * expected to commit E = 1 + sum of their P tokens (the accepted path plus the
 * model's own token), and costs us_by_rows[n] (n + 1 rows: the kept nodes and
 * the root). The candidate with the largest E / time wins; equal rates keep
 * the smaller tree.
 * Outputs: *n_keep, keep[n_nodes] (1 = kept), and if not NULL the winner's
 * *expected_tokens and *tokens_per_ms.
 * Errors: INVALID_ARG (null pointer, p outside [0, 1] or NaN, children's
 * probabilities summing above 1, a price that is not positive and finite),
 * SHAPE (n_nodes outside 1..NVFP4V_STAIRCUT_MAX_NODES, a parent that does not
 * precede its child, a candidate < 1), M_RANGE (a candidate needs more rows
 * than max_rows). */
#define NVFP4V_STAIRCUT_MAX_NODES 4096
int nvfp4v_staircut(const double *us_by_rows, int max_rows, const int32_t *parent,
                    const double *p_accept, int n_nodes, const int32_t *sizes, int n_sizes,
                    int32_t *n_keep, uint8_t *keep, double *expected_tokens,
                    double *tokens_per_ms);

/* ---- Full verify pass (chained layer stack) ----------------------------- */

/* One layer of the dense stand-in stack. The pages give neither layer shapes
 * nor the non-GEMM operations of the model (TandemLLM manual, "What TandemLLM
 * is", 1.2 "Two levers"; 1.4 "What runs today"), so the pass is a uniform
 * stack of the projections a dense layer streams, each packed with
 * nvfp4v_pack:
 *   qkv     [3H x H]  q, k and v stacked along N (rows 0..H-1 are q, ...)
 *   o       [H x H]
 *   gate_up [2I x H]  gate and up interleaved in 16-row tiles: packed rows
 *                     32t..32t+15 are gate rows 16t..16t+15 and rows
 *                     32t+16..32t+31 are up rows 16t..16t+15
 *   down    [H x I]
 * with one fp32 tensor scale per packed matrix. */
typedef struct nvfp4v_layer {
  const void *qkv;
  const void *o;
  const void *gate_up;
  const void *down;
  float ts_qkv, ts_o, ts_gate_up, ts_down;
} nvfp4v_layer;

/* Elementwise chain glue, fp32 arithmetic, result rounded to bf16 (nearest
 * even); x/y are fp32 [rows][ld], out is bf16 [rows][cols] (dense).
 *   glue_scale: out = bf16(x * c)
 *   glue_sum:   out = bf16(x * c + y * c)   (no fused multiply-add) */
int nvfp4v_glue_scale(nvfp4v_ctx *ctx, const float *x_dev, int64_t ldx, int64_t rows, int64_t cols,
                      float c, uint16_t *out_dev, hipStream_t stream);
int nvfp4v_glue_sum(nvfp4v_ctx *ctx, const float *x_dev, int64_t ldx, const float *y_dev,
                    int64_t ldy, int64_t rows, int64_t cols, float c, uint16_t *out_dev,
                    hipStream_t stream);

/* Bytes of caller-owned device workspace nvfp4v_verify_pass needs for
 * n_layers layers (0 for bad arguments): the fp32 outputs of one layer plus
 * one block of packed activations (both copies) per layer and GEMM (about
 * 2 MiB per layer at M = 16, H = 5120, I = 17408). */
size_t nvfp4v_pass_workspace_bytes(int64_t m, int64_t hidden, int64_t inter, int n_layers);

/* How nvfp4v_verify_pass schedules its GEMMs (per context; default CHAIN):
 *   NVFP4V_PASS_CHAIN       one GEMM launch per projection, four per layer,
 *                           stream-ordered;
 *   NVFP4V_PASS_PERSISTENT  one cooperatively launched persistent kernel per
 *                           32 layers whose work-groups meet at a grid barrier
 *                           between dependent GEMMs.
 * Both modes are deterministic (equal inputs give equal bits on every call);
 * at some shapes they split K differently, so their fp32 sums can differ in
 * the last bits.
 * Errors: INVALID_ARG. */
#define NVFP4V_PASS_CHAIN 0
#define NVFP4V_PASS_PERSISTENT 1
int nvfp4v_set_pass_mode(nvfp4v_ctx *ctx, int mode);
int nvfp4v_get_pass_mode(const nvfp4v_ctx *ctx);

/* Enqueue the whole pass on `stream`: one packing kernel, then the layers'
 * GEMMs as the context's pass mode schedules them. For each layer, with c_h = H^-1/2,
 * c_2 = (2H)^-1/2 and c_i = I^-1/2 (fp32, rounded from fp64):
 *   qkv = GEMM(h, qkv);          o_in = glue_scale(v part of qkv, c_h)
 *   o   = GEMM(o_in, o);         g_in = glue_scale(o, c_h)
 *   gu  = GEMM(g_in, gate_up);   d_in = glue_sum(gate part, up part, c_2)
 *   d   = GEMM(d_in, down);      h    = glue_scale(d, c_i)
 * h0 is bf16 [M][H]; the last layer's h goes to h_out (bf16 [M][H]). If trace
 * is not NULL, layer l's output h is also copied to trace[l][M][H]. Every
 * glue map is linear, so activations keep an O(1) RMS over the stack. Each
 * glue step runs in the epilogue of the GEMM that produces its input; fp32
 * outputs are written for the last layer only (earlier ones would be
 * overwritten unread). In
 * the persistent mode a barrier wait that exceeds 2 s (it cannot while the launch
 * is co-resident) ends the kernel early and sets an error flag that
 * nvfp4v_pass_status reports; the outputs are then undefined. After the call returns, the
 * workspace holds the last layer's fp32 GEMM outputs (qkv [M][3H] at offset 0,
 * then o [M][H], gu [M][2I] with gate columns 0..I-1 and up columns I..2I-1,
 * d [M][H], each 256-byte aligned). For M > 64 the workspace is one such
 * region per block of 64 rows, in row order: block b (rows 64 b ..) starts at
 * b * nvfp4v_pass_workspace_bytes(64, hidden, inter, n_layers) and holds its
 * own rows only.
 * Does not allocate or synchronise. Calls on one context must not overlap.
 * Errors: INVALID_ARG, SHAPE (H or I not a multiple of 16), M_RANGE, ALIGN,
 * WORKSPACE, HIP, FAULT. */
int nvfp4v_verify_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t hidden,
                       int64_t inter, const uint16_t *h0_dev, int64_t m, void *ws_dev,
                       size_t ws_bytes, uint16_t *h_out_dev, uint16_t *trace_dev,
                       hipStream_t stream);

/* Synchronise the device and report whether the last persistent pass on this
 * context finished (NVFP4V_OK) or gave up at a barrier (NVFP4V_E_TIMEOUT). */
int nvfp4v_pass_status(nvfp4v_ctx *ctx);
/* Synchronise and return where the last persistent pass gave up: 0 if it did
 * not, 1 at a grid barrier. For diagnosis; nvfp4v_pass_status reports the
 * failure itself. Errors: INVALID_ARG, HIP. */
int nvfp4v_pass_error_site(nvfp4v_ctx *ctx);
/* Work-groups of the last persistent pass launch (0 before the first). */
int nvfp4v_last_pass_grid(const nvfp4v_ctx *ctx);
/* Phase timeline of the last pass, for profiling (only when the context was
 * created with NVFP4V_PASS_TRACE=1 in the environment, else INVALID_ARG):
 * synchronously copies up to max_words words into out_host, laid out as
 * [phase][1024 work-group slots][2]: the 100 MHz real-time clock when the
 * work-group started the phase and when it finished its work in it (before
 * the barrier). *phases and *groups receive the phase and work-group counts. */
int nvfp4v_pass_timeline(nvfp4v_ctx *ctx, uint64_t *out_host, size_t max_words, int *phases,
                         int *groups);

/* ---- Measurement helpers ------------------------------------------------- */

/* Stream `bytes` (multiple of 16, 16-byte aligned) from HBM with 16-byte loads
 * and fold them into sink_dev (nvfp4v_read_probe_sink_words() words): the
 * practical read ceiling the GEMM's bandwidth is compared with. */
size_t nvfp4v_read_probe_sink_words(nvfp4v_ctx *ctx);
int nvfp4v_read_probe(nvfp4v_ctx *ctx, const void *buf_dev, size_t bytes, uint32_t *sink_dev,
                      hipStream_t stream);
/* Plain device copy of `bytes` (a kernel of known traffic, for calibrating
 * hardware byte counters). */
int nvfp4v_copy_probe(nvfp4v_ctx *ctx, const void *src_dev, void *dst_dev, size_t bytes,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4V_H */
