/*
 * vbq.h -- C ABI of libvbq.so, the MI355X (gfx950) decode path of Variable
 * Bit-width Quantization (VBQ).
 *
 * Method ("Variable Bit-width Quantization", mlsanity.com page, Abstract):
 * every contiguous group of 64 weights carries its own bit-width from
 * {1, 2, 4, 8}; the frozen allocation is stored as packed low-bit codes and
 * autoregressive decode, which is memory-bandwidth bound, multiplies them
 * with fused dequantize-and-multiply kernels.  The pages fix neither the
 * dequant rule nor the storage; this library fixes them as follows:
 *
 *   - one fp16 scale s per group; code q in [0, 2^b - 1];
 *     w = s * (q - (2^b - 1)/2), exact in fp32 for every finite s;
 *   - groups run along K (the reduction axis); K % 64 == 0;
 *   - packed layout "VBQ1", byte for byte:
 *       header (256 B): u32 magic 0x31514256, version 1, N, K, G=K/64,
 *         S=32 (groups per K-slice), nS=ceil(G/32), row_pad=128; u64 section
 *         offsets row_off, slice_off, wmap, scales, codes; u64 total_bytes,
 *         code_bytes (sum of 8*b), code_bytes_padded; zeros to byte 255.
 *       sections at 256-byte aligned offsets:
 *         row_off   u32[N+1]     row n's code record start, 128-byte units
 *         slice_off u32[N][nS]   byte offset of slice t in row n's record
 *         wmap      u32[N][nS][2] bit planes of log2(b) for groups 32t+i
 *         scales    u16[N][G]    fp16 bits, natural order
 *         codes     per-row records padded with zeros to 128 B; inside a
 *                   slice, groups are bucketed by width (1,2,4,8), ascending
 *                   g in a bucket, 8*b bytes per group
 *       group encoding: halves H0 = codes 0..31 and H1 = codes 32..63 are
 *         packed LSB-first into 16-bit units (code j at bit j*b of its half);
 *         32-bit word d = H0 unit d | H1 unit d << 16.
 *
 * Conventions for every call below:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     memory (blob, q, bits, scales, x, y, w, workspaces, status words).  The
 *     library allocates no device memory at run time; its only global state
 *     is (a) a per-(kernel, device) record that the dynamic-LDS attribute has
 *     been set (mutex-guarded, set on a kernel's first launch on a device),
 *     (b) vbq_last_error()'s thread-local text, and (c) the 256-byte device
 *     array of vbq_gemv_planned_argmax_noalloc, one per device that calls it.
 *     The compute-unit count is read from the current device on every call.
 *   - Calls are asynchronous on `stream` unless marked SYNC.  Argument checks
 *     run on the host before any launch; a call that returns an error has
 *     launched nothing.  VBQ_ERR_HIP carries the HIP error text in
 *     vbq_last_error().
 *   - Calls are reentrant.  Calls that share a workspace must be ordered (same
 *     stream); concurrent calls need distinct workspaces.
 */
#ifndef VBQ_H
#define VBQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vbq_status {
    VBQ_OK = 0,
    VBQ_ERR_INVALID_ARG = 1, /* null pointer, bad enum */
    VBQ_ERR_SHAPE = 2,       /* N < 1, K < 64, K % 64 != 0, ld too small */
    VBQ_ERR_BATCH = 3,       /* M outside [1, 16] */
    VBQ_ERR_BITS = 4,        /* a width outside {1, 2, 4, 8} */
    VBQ_ERR_CODE_RANGE = 5,  /* a code q > 2^b - 1 */
    VBQ_ERR_ALIGN = 6,       /* blob not 256-byte aligned, or x/y/w not element aligned */
    VBQ_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
    VBQ_ERR_LAYOUT = 8,      /* bad magic/version/sizes, or blob inconsistent with its widths */
    VBQ_ERR_HIP = 9          /* a HIP runtime call failed */
} vbq_status;

typedef enum vbq_dtype { VBQ_F32 = 0, VBQ_F16 = 1 } vbq_dtype;

/* Host mirror of bytes 0..95 of the blob header. */
typedef struct vbq_layout {
    uint32_t magic, version, N, K, G, S, nS, row_pad;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    uint64_t total_bytes, code_bytes, code_bytes_padded;
} vbq_layout;

/* Device status-word bits set by vbq_pack, vbq_quantize and vbq_prepare
 * (read with vbq_status_check). */
#define VBQ_STATUS_BITS 0x1u   /* some width outside {1,2,4,8} */
#define VBQ_STATUS_CODES 0x2u  /* some code above 2^b - 1 */
#define VBQ_STATUS_LAYOUT 0x4u /* widths disagree with the planned layout */
#define VBQ_STATUS_PLAN 0x8u   /* a row block needs more passes than its plan holds */

/* Library version string, e.g. "vbq 0.1.0 (VBQ1 layout)". */
const char *vbq_version(void);

/* Static text for a status code. */
const char *vbq_status_string(vbq_status st);

/* Text of the last HIP error seen by this thread ("" if none). */
const char *vbq_last_error(void);

/*
 * Host only.  Fill the shape-dependent fields of a layout (dims and section
 * offsets); the code sizes and total_bytes need the widths (vbq_pack_plan).
 */
vbq_status vbq_layout_init(int N, int K, vbq_layout *L /* host */);

/*
 * Host only.  Validate a blob header copied to the host (>= 256 bytes) and
 * return its layout.  VBQ_ERR_LAYOUT on a bad magic, version or geometry.
 */
vbq_status vbq_layout_from_header(const void *header /* host, 256 B */, vbq_layout *L /* host */);

/* Workspace bytes vbq_pack_plan needs for N rows. */
size_t vbq_pack_plan_workspace(int N);

/*
 * SYNC.  Plan a blob for widths bits[N][G] (u8, device): computes the per-row
 * 128-byte-padded record sizes and fills L completely (total_bytes is what
 * the caller must allocate).  Returns VBQ_ERR_BITS if any width is invalid.
 * ws: device scratch of vbq_pack_plan_workspace(N) bytes, any contents.
 */
vbq_status vbq_pack_plan(int N, int K, const uint8_t *bits, vbq_layout *L /* host */, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Storage of the frozen allocation: "Variable Bit-width Quantization"
 * (mlsanity.com page, Abstract) keeps each 64-weight group at its own width
 * in {1, 2, 4, 8} and stores the model as packed low-bit codes; the VBQ1
 * layout above is this library's packing of them.
 * Pack q[N][K] (u8 codes), bits[N][G] (u8 widths), scales[N][G] (fp16 bits)
 * into blob (L->total_bytes bytes, 256-byte aligned, any prior contents).
 * Every blob byte is written; the result is the unique VBQ1 byte string.
 * Data errors found on the device (bad width, code out of range, widths that
 * differ from the plan) set VBQ_STATUS_* bits in *status_word (device u32,
 * cleared by this call); no write ever leaves [blob, blob + total_bytes).
 */
vbq_status vbq_pack(const vbq_layout *L /* host */, const uint8_t *q, const uint8_t *bits, const uint16_t *scales,
                    void *blob, uint32_t *status_word, hipStream_t stream);

/*
 * SYNC.  Read a status word written by vbq_pack, vbq_quantize or vbq_prepare:
 * VBQ_OK, or the first error among VBQ_ERR_BITS, VBQ_ERR_CODE_RANGE,
 * VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE (VBQ_STATUS_PLAN).  *raw (host, may be NULL)
 * receives the word.
 */
vbq_status vbq_status_check(const uint32_t *status_word, uint32_t *raw /* host */, hipStream_t stream);

/*
 * Round-to-nearest codes and scales for a given width map: the step before
 * vbq_pack.  "Variable Bit-width Quantization" (mlsanity.com page, Abstract)
 * gives every group of 64 weights its own width in {1, 2, 4, 8} and learns
 * its scales in training; the pages give no rule turning float weights into
 * codes, and this call implements the plain one.  Per group of row n, columns
 * 64g..64g+63, width b = bits[n][g], c = (2^b - 1) / 2:
 *   a = max |w| (fp32; NaN weights are skipped),  s = fp16_rne(a / c),
 *   q = min(max(rint(w / s + c), 0), 2^b - 1)  (fp32 operations, rint ties to
 *   even; a NaN quotient gives 0, so an all-zero group gets s = 0, q = 0).
 * w: device [N][ldw] (ldw >= K) of wt (VBQ_F32, or VBQ_F16 widened exactly);
 * bits: device u8 [N][G]; q: device u8 [N][K] (out, 8-byte aligned); scales:
 * device fp16 bits [N][G] (out).  A width outside {1, 2, 4, 8} gives that group q = 0 and
 * s = 0 and sets VBQ_STATUS_BITS in *status_word (device u32, cleared by this
 * call; may be NULL).  Errors: VBQ_ERR_INVALID_ARG, VBQ_ERR_SHAPE (N < 1,
 * K % 64, ldw < K), VBQ_ERR_ALIGN, VBQ_ERR_HIP.
 */
vbq_status vbq_quantize(int N, int K, const void *w, vbq_dtype wt, int ldw, const uint8_t *bits, uint8_t *q,
                        uint16_t *scales, uint32_t *status_word, hipStream_t stream);

/*
 * The dequantize half of the fused dequantize-and-multiply kernels of
 * "Variable Bit-width Quantization" (mlsanity.com page, Abstract), on its own:
 * the group rule w = s * (q - (2^b - 1)/2) stated at the top of this file.
 * Expand a blob to dense weights w[N][K] (row-major): VBQ_F32 gives the exact
 * value of s*(q - (2^b-1)/2); VBQ_F16 gives its round-to-nearest-even fp16.
 */
vbq_status vbq_dequant(const vbq_layout *L /* host */, const void *blob, void *w, vbq_dtype wt, hipStream_t stream);

/*
 * Workspace bytes vbq_gemv / vbq_gemv_batched can use for layout L and M
 * tokens (1 <= M <= 32) on the current device: 0 for M <= 2 when K <= 16256
 * (the streaming kernel); otherwise the fp32 partial
 * sums ([segments][M][N]) of the K segments the matrix-core kernel cuts a
 * matrix with few row blocks into (0 when it cuts none).  The workspace is
 * optional: with at least this many bytes (4-byte aligned) each segment runs as
 * its own workgroups and a second kernel adds the partial sums; with less, or
 * NULL, one workgroup per row block runs all segments and adds their sums in
 * the same order, so the result is the same bit for bit, only slower.
 */
vbq_status vbq_workspace_size(const vbq_layout *L /* host */, int M, size_t *bytes /* host */);

/* Zero-fill a GEMV workspace with a kernel (safe inside HIP graph capture). */
vbq_status vbq_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The decode GEMV: "Variable Bit-width Quantization" (mlsanity.com page,
 * Abstract) decodes autoregressively, bound by memory bandwidth, with fused
 * dequantize-and-multiply kernels over the packed mixed-width codes; this is
 * that product for one token, read straight from a VBQ1 blob.
 * y = W x for one token: x fp16[K], y[N] in yt (VBQ_F16 rounds to nearest
 * even).  Accumulation is fp32; |y - y_exact| <= 1e-3 * sum_k |w_k||x_k| per
 * output.  Outputs that meet a non-finite weight (inf/NaN scale) with a
 * nonzero x are non-finite.  Same as vbq_gemv_batched with M = 1.
 */
vbq_status vbq_gemv(const vbq_layout *L /* host */, const void *blob, const uint16_t *x, void *y, vbq_dtype yt,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same fused dequantize-and-multiply product ("Variable Bit-width
 * Quantization", mlsanity.com page, Abstract) for a decode batch of M tokens.
 * Y = X W^T for M tokens (1 <= M <= 32): x fp16 [M][ldx] (ldx >= K),
 * y [M][ldy] (ldy >= N).  Each packed code is unpacked once per call and
 * reused for all M tokens.  Error bound as vbq_gemv, per token and output.
 * For 3 <= M <= 32 with x 16-byte aligned and ldx % 8 == 0 the product runs on
 * the matrix cores (fp16 operands exact, fp32 accumulation, one or two tiles
 * of 16 tokens per call); a token's outputs then do not depend on the other
 * tokens of the batch or on M, bit for bit.  M <= 2 runs on the vector units
 * (one streaming kernel) when K <= 16256, else also on the matrix cores when x
 * and ldx allow it.  M > 16 runs only there:
 * VBQ_ERR_ALIGN when x or ldx does not meet those conditions, VBQ_ERR_SHAPE
 * when the blob or the span of x exceeds 4 GiB.
 * ws / ws_bytes: optional, see vbq_workspace_size (results do not depend on
 * it); calls sharing a workspace must be ordered.
 */
vbq_status vbq_gemv_batched(const vbq_layout *L /* host */, const void *blob, int M, const uint16_t *x, int ldx,
                            void *y, int ldy, vbq_dtype yt, void *ws, size_t ws_bytes, hipStream_t stream);

/* One matrix of a vbq_gemv_shared call. */
typedef struct vbq_gemv_item {
    const vbq_layout *L; /* host */
    const void *blob;    /* device, 256-byte aligned, from vbq_pack */
    void *y;             /* device, [M][ldy] in the call's yt */
    int ldy;             /* >= L->N */
} vbq_gemv_item;

#define VBQ_MAX_SHARED 4

/*
 * y_i = W_i x for n (1..VBQ_MAX_SHARED) matrices with the same K that read the
 * same activations x [M][ldx] (1 <= M <= 16): the fused dequantize-and-multiply
 * of "Variable Bit-width Quantization" (mlsanity.com page, Abstract) applied to
 * projections that share their input, such as the gate and up projections of a
 * SwiGLU MLP block.  For M <= 2 the matrices run in ONE launch that stages x
 * once; otherwise (or for shapes the streaming kernel does not take) they are
 * launched one after another.  Items and layouts are host memory read during
 * the call; x and the y_i are device memory owned by the caller.  Each y_i
 * obeys the vbq_gemv error bound.  Errors: VBQ_ERR_INVALID_ARG (null pointers,
 * n out of range, yt), VBQ_ERR_BATCH (M), VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE
 * (different K, ldx < K, ldy < N), VBQ_ERR_ALIGN; nothing is launched then.
 */
vbq_status vbq_gemv_shared(const vbq_gemv_item *items /* host */, int n, int M, const uint16_t *x, int ldx,
                           vbq_dtype yt, hipStream_t stream);

/*
 * Prepared plans.  vbq_gemv reads the VBQ1 blob directly and must work out, at
 * run time and per tile, which groups have which width before a wavefront can
 * run 64 groups of one width ("Variable Bit-width Quantization", mlsanity.com
 * page, Abstract: each 64-weight group carries its own width).  A plan does
 * that once per matrix: a device copy of the blob's codes and scales,
 * re-ordered for the GEMV kernel of this library on this device.
 *
 * Plan buffer: `wgs` row blocks of `rows` rows (the last may have fewer), one
 * per workgroup of the GEMV launch.  Block b owns bytes [b * region_bytes,
 * (b + 1) * region_bytes).  Its groups are sorted by (width 1, 2, 4, 8; then
 * column; then row) and cut into passes of 1 KiB of codes: 128 one-bit, 64
 * two-bit, 32 four-bit or 16 eight-bit groups (the last pass of a width may be
 * partly filled).  Pass p of a block is the 1536-byte record at p * 1536:
 *   bytes [0, 1024): group k's code record (8*b bytes, copied verbatim from
 *     the blob) at k * 8*b;
 *   bytes [1024, 1536): the word of group k, fp16 scale bits | e << 16, in
 *     the 2^c u32 slots k 2^c .. (k + 1) 2^c - 1 (c = log2(b): one slot for a
 *     one-bit group, 2, 4 or 8 copies otherwise, so the 512 bytes are full and
 *     the 8 bytes GEMV lane l loads hold the words of the groups it works on);
 *     e = column * S + (row - first row of the block); the position
 *     stride S = max(rows, 2) below 32 rows, else the smallest S >= rows with
 *     S = 64 / L (mod 32), L = 8, 16, 32 or 64 for G <= 64, <= 128, <= 256 or
 *     more;
 *   an empty place of a partly filled pass has zero codes and the word
 *     (S * G) << 16 (scale 0 at a position no row uses).
 * After the `passes` records (at passes * 1536): the width byte of each pass
 * (log2(b) + 1; 0 after the block's last pass), wave-major for the 16
 * wavefronts of the GEMV workgroup: pass w + 16 j at byte w * per_wave + j;
 * per_wave = ceil(passes / 16) + 1 rounded up to a multiple of 4, so every
 * wavefront's list ends with a 0.  region_bytes = passes * 1536 +
 * 16 * per_wave rounded up to 256.  Bytes of a region past what its block
 * uses are never read for arithmetic.
 */
#define VBQ_PLAN_MAGIC 0x33504256u

typedef struct vbq_plan {
    uint32_t magic;        /* VBQ_PLAN_MAGIC */
    int32_t N, K, G;       /* matrix shape (G = K / 64 <= 512) */
    int32_t M;             /* tokens per GEMV launch (1 or 2) */
    int32_t wgs, rows;     /* row blocks (workgroups) and rows per block */
    int32_t passes;        /* pass records per block region (the largest block's count) */
    int32_t per_wave;      /* width bytes per wavefront */
    int32_t psum;          /* partial sums per token a block needs in LDS */
    int32_t lds_bytes;     /* LDS per workgroup of its GEMV launches */
    int32_t reserved;
    uint64_t region_bytes; /* bytes per block region */
    uint64_t total_bytes;  /* plan buffer bytes: wgs * region_bytes */
} vbq_plan;

/*
 * SYNC.  Fill *P for the matrix (L, blob) and launches of up to M tokens (1
 * or 2).  `wgs` row blocks (<= 0: one per compute unit of the current
 * device); the rows per block are even whenever N is even, and the block
 * count grows where a block's partial sums would not fit the LDS of one
 * workgroup (P->M comes back as 1 when two tokens would need more than four
 * blocks per compute unit).  GEMVs of more tokens run as several launches
 * over the same plan.  Runs one sizing kernel over the width bit planes
 * (workspace ws: device, >= 16 bytes) and waits for it.  Errors:
 * VBQ_ERR_INVALID_ARG, VBQ_ERR_LAYOUT, VBQ_ERR_BATCH (M), VBQ_ERR_WORKSPACE,
 * VBQ_ERR_ALIGN, VBQ_ERR_SHAPE (K > 32768, or no block size fits the LDS),
 * VBQ_ERR_HIP.
 */
vbq_status vbq_plan_init(const vbq_layout *L /* host */, const void *blob, int M, int wgs, vbq_plan *P /* host */,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Write the plan of (L, blob) described by *P into `plan` (device,
 * P->total_bytes, 256-byte aligned).  The blob must be the one *P was sized
 * for: a row block that would need more passes than P->passes is not written
 * and sets VBQ_STATUS_PLAN in *status_word (device u32, 4-byte aligned,
 * cleared by this call; may be NULL).  Errors: VBQ_ERR_INVALID_ARG,
 * VBQ_ERR_LAYOUT (bad *P), VBQ_ERR_SHAPE (P does not match L), VBQ_ERR_ALIGN.
 */
vbq_status vbq_prepare(const vbq_plan *P /* host */, const vbq_layout *L /* host */, const void *blob, void *plan,
                       uint32_t *status_word, hipStream_t stream);

/*
 * Y = X W^T from a plan, M tokens (1 <= M <= 16): x fp16 [M][ldx] (ldx >= K),
 * y [M][ldy] (ldy >= N) in yt.  Same results contract as vbq_gemv_batched
 * (fp32 accumulation, |y - y_exact| <= 1e-3 * sum_k |w_k||x_k|), and the
 * result does not depend on timing: token m's outputs are bit-identical for
 * every M.  One launch of P->wgs workgroups per P->M tokens.
 * Errors: VBQ_ERR_INVALID_ARG, VBQ_ERR_LAYOUT, VBQ_ERR_BATCH, VBQ_ERR_SHAPE,
 * VBQ_ERR_ALIGN (plan not 256-byte aligned, x/y not element aligned).
 */
vbq_status vbq_gemv_planned(const vbq_plan *P /* host */, const void *plan, int M, const uint16_t *x, int ldx,
                            void *y, int ldy, vbq_dtype yt, hipStream_t stream);

/*
 * Greedy-decode epilogue for the LM head ("Variable Bit-width Quantization",
 * mlsanity.com page, Abstract: the quantized models decode autoregressively;
 * greedy decoding takes the token of the largest logit).  Workspace of
 * vbq_gemv_planned_argmax: key/count are internal and must be zero before the
 * first call (e.g. hipMemset once); every call leaves them zero again.
 */
typedef struct vbq_argmax_ws {
    uint64_t key[16];     /* internal */
    uint32_t count;       /* internal */
    uint32_t reserved[3];
    int32_t index[16];    /* out: token m's row of the largest output */
    float value[16];      /* out: that output, fp32 */
} vbq_argmax_ws;

/*
 * For each token m < M (1..16): the row n of the largest y[m][n] of
 * Y = X W^T from a plan, without writing Y.  Values are the fp32 outputs of
 * vbq_gemv_planned (bit for bit), ordered by the IEEE total order
 * (-NaN < -inf < ... < +inf < +NaN); ties go to the smallest row.  One launch
 * per P->M tokens; the last workgroup of each launch writes index/value of its
 * tokens into ws (device, 8-byte aligned).  Calls sharing a workspace must be
 * ordered (one stream).  Errors: VBQ_ERR_INVALID_ARG, VBQ_ERR_BATCH,
 * VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE, VBQ_ERR_ALIGN.
 */
vbq_status vbq_gemv_planned_argmax(const vbq_plan *P /* host */, const void *plan, int M, const uint16_t *x,
                                   int ldx, vbq_argmax_ws *ws, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): the result of
 * vbq_gemv_planned_argmax (the same launches, bit for bit) with no workspace
 * argument.  The keys and the ticket counter live in a 256-byte device array
 * of the library (one per device, held until the process ends, cleared by
 * the first call on each device, left cleared by every call); token m's row
 * of the largest output goes to index[m] and that output to value[m] (device,
 * 4-byte aligned, M entries each).  Calls on one device share the array:
 * calls that overlap on a device (different streams) race and must be
 * ordered by the caller.  No device memory is allocated.  Errors:
 * VBQ_ERR_INVALID_ARG, VBQ_ERR_BATCH (M outside [1, 16], the array's
 * limit), VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE, VBQ_ERR_ALIGN, VBQ_ERR_HIP.
 */
vbq_status vbq_gemv_planned_argmax_noalloc(const vbq_plan *P /* host */, const void *plan, int M, const uint16_t *x,
                                           int ldx, int32_t *index, float *value, hipStream_t stream);

/*
 * SwiGLU epilogue for the gate and up projections of an MLP block, which read
 * the same activations (the decode path of "Variable Bit-width Quantization",
 * mlsanity.com page, Abstract, runs the model's projections as fused
 * dequantize-and-multiply GEMVs).  The plan is of ONE matrix of 2N rows with
 * the gate and up rows interleaved (row 2i = gate row i, row 2i+1 = up row i;
 * the caller packs it so); its plan must have an even row count per block,
 * which vbq_plan_init gives whenever the row count is even.  Writes, for
 * tokens m < M (1..16), h[m][i] = silu(g) * u with g, u the fp32 outputs of
 * rows 2i, 2i+1 (silu(g) = g / (1 + exp(-g)) in fp32), h [M][ldh]
 * (ldh >= N) in ht, without writing the 2N projections.  Errors:
 * VBQ_ERR_INVALID_ARG, VBQ_ERR_BATCH, VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE (odd row
 * count or rows per block, ldh < N), VBQ_ERR_ALIGN.
 */
vbq_status vbq_gemv_planned_swiglu(const vbq_plan *P /* host */, const void *plan, int M, const uint16_t *x,
                                   int ldx, void *h, int ldh, vbq_dtype ht, hipStream_t stream);

/* One matrix of a vbq_gemv_planned_shared call. */
typedef struct vbq_planned_item {
    const vbq_plan *P; /* host */
    const void *plan;  /* device, from vbq_prepare */
    void *y;           /* device, [M][ldy] in the call's yt */
    int ldy;           /* >= P->N */
} vbq_planned_item;

/*
 * vbq_gemv_planned for n (1..VBQ_MAX_SHARED) matrices that read the same x
 * (e.g. the gate and up projections of one MLP block), in ONE launch of
 * max P_i->wgs x n workgroups.  The plans must agree on K, and the partial
 * sums of the largest block must fit one workgroup's LDS (VBQ_ERR_SHAPE
 * otherwise); prepare them with the same M and with wgs in proportion to N
 * so that the launch spans the device once.
 */
vbq_status vbq_gemv_planned_shared(const vbq_planned_item *items /* host */, int n, int M, const uint16_t *x, int ldx,
                                   vbq_dtype yt, hipStream_t stream);

/*
 * Decode-step executors.  Autoregressive decode ("Variable Bit-width
 * Quantization", mlsanity.com page, Abstract) runs a model's projections in a
 * fixed order, each reading activations the previous stage produced.  A step
 * is given as an array of GEMVs tagged with a stage number (non-decreasing
 * along the array, at most 1024 items per stage) and enqueued on `stream` in
 * that order, so the stream completes every stage before the next starts.
 * Inside a stage, items that read the same x (same pointer and ldx) with the
 * same K run as shared launches of up to VBQ_MAX_SHARED matrices; the others
 * run one launch each.  Every item's y obeys the vbq_gemv error bound and
 * equals what the single-matrix call gives for it.  Items are host memory read
 * during the call; every pointer inside is device memory owned by the caller.
 * Every item is checked before the first launch: a call that returns an error
 * has launched nothing.  Errors: VBQ_ERR_INVALID_ARG (null pointers, n < 1,
 * yt, stages decreasing or a stage over 1024 items), VBQ_ERR_BATCH (M outside
 * [1, 16]), VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE, VBQ_ERR_ALIGN, VBQ_ERR_HIP.
 * Capturing the call in a HIP graph captures the whole step.
 */
typedef struct vbq_seq_item {
    const vbq_layout *L; /* host */
    const void *blob;    /* device, 256-byte aligned, from vbq_pack */
    const uint16_t *x;   /* device, fp16 [M][ldx] */
    int ldx;             /* >= L->K */
    void *y;             /* device, [M][ldy] in the call's yt */
    int ldy;             /* >= L->N */
    int stage;
} vbq_seq_item;

/* The step over packed blobs: each launch as vbq_gemv_batched / vbq_gemv_shared
 * would make it.  ws / ws_bytes are passed to every GEMV (NULL / 0 is valid,
 * see vbq_workspace_size). */
vbq_status vbq_gemv_seq(const vbq_seq_item *items /* host */, int n, int M, vbq_dtype yt, void *ws, size_t ws_bytes,
                        hipStream_t stream);

typedef struct vbq_planned_seq_item {
    const vbq_plan *P;  /* host */
    const void *plan;   /* device, from vbq_prepare */
    const uint16_t *x;  /* device, fp16 [M][ldx] */
    int ldx;            /* >= P->K */
    void *y;            /* device, [M][ldy] in the call's yt */
    int ldy;            /* >= P->N */
    int stage;
} vbq_planned_seq_item;

/* The step over prepared plans: each launch as vbq_gemv_planned_shared would
 * make it.  Items of a stage share a launch when they read the same x, their
 * plans agree on K and M, and one workgroup's LDS holds the partial sums of
 * the largest of their blocks. */
vbq_status vbq_gemv_planned_seq(const vbq_planned_seq_item *items /* host */, int n, int M, vbq_dtype yt,
                                hipStream_t stream);

/*
 * Prefill GEMM.  With many tokens (M > 16: a prompt's tokens, or a large
 * batch) Y = X W^T is a dense contraction over K, unlike decode; this path
 * runs it on the matrix cores.  Each 64-weight group keeps its own width from
 * {1, 2, 4, 8} ("Variable Bit-width Quantization", mlsanity.com page,
 * Abstract); a GEMM plan re-orders the blob once per matrix so that tiles of
 * the weights can be dequantized to fp16 in LDS by wavefronts that each take
 * groups of one width.
 *
 * GEMM plan buffer:
 *   u32 offset table [nb * kc + 1]: tile (row block i, column chunk j) starts
 *     at 16 * table[i * kc + j] bytes from the buffer start; entry nb * kc is
 *     the end of the last tile; zeros up to table_bytes (a multiple of 256).
 *   tiles, row-block major: rows 128 i .. 128 i + 127 (fewer in the last
 *     block), columns 128 j .. 128 j + 127 (groups 2 j, 2 j + 1; one in the
 *     last chunk of an odd G).  A tile is
 *       16-byte header: u16 groups of width 8, 4, 2, 1; u32 tile bytes; u32
 *         offset of the word section;
 *       code records (8*b bytes each, copied verbatim from the blob) in slot
 *         order: width 8, 4, 2, 1, then column, then row;
 *       u32 per group in slot order: fp16 scale bits | (column * 128 + row) << 16
 *         (column and row inside the tile);
 *       zeros to a multiple of 16 bytes.
 *   zeros: slot_bytes of padding after the last tile.
 */
#define VBQ_GEMM_PLAN_MAGIC 0x4D4D4756u

typedef struct vbq_gemm_plan {
    uint32_t magic;        /* VBQ_GEMM_PLAN_MAGIC */
    int32_t N, K, G;       /* matrix shape (K <= 32768) */
    int32_t nb, kc;        /* row blocks of 128 rows, column chunks of 128 columns */
    int32_t max_tile;      /* bytes of the largest tile */
    int32_t slot_bytes;    /* max_tile rounded up to 4 KiB (LDS slot of the GEMM kernel) */
    uint64_t table_bytes;  /* bytes of the offset table (multiple of 256) */
    uint64_t total_bytes;  /* plan buffer bytes */
} vbq_gemm_plan;

/*
 * SYNC.  Fill *P for the matrix (L, blob): one sizing kernel over the width
 * bit planes (workspace ws: device, >= 16 bytes, 8-byte aligned), then a wait.
 * Errors: VBQ_ERR_INVALID_ARG, VBQ_ERR_LAYOUT, VBQ_ERR_WORKSPACE,
 * VBQ_ERR_ALIGN (blob not 256-byte aligned), VBQ_ERR_SHAPE (K > 32768),
 * VBQ_ERR_HIP.
 */
vbq_status vbq_gemm_plan_init(const vbq_layout *L /* host */, const void *blob, vbq_gemm_plan *P /* host */,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Write the GEMM plan of (L, blob) described by *P into buf (device,
 * P->total_bytes, 256-byte aligned); every byte of buf is written.  The blob
 * must be the one *P was sized for: if its tiles do not fit (a tile larger
 * than P->max_tile, or more tile bytes than the buffer holds), no tile is
 * written past the buffer, the plan is unusable and VBQ_STATUS_PLAN is set in
 * *status_word (device u32, 4-byte aligned, cleared by this call; may be
 * NULL).  Errors: VBQ_ERR_INVALID_ARG, VBQ_ERR_LAYOUT, VBQ_ERR_SHAPE (P does
 * not match L), VBQ_ERR_ALIGN.
 */
vbq_status vbq_gemm_prepare(const vbq_gemm_plan *P /* host */, const vbq_layout *L /* host */, const void *blob,
                            void *buf, uint32_t *status_word, hipStream_t stream);

/* Workspace bytes vbq_gemm needs for M tokens on the current device. */
vbq_status vbq_gemm_workspace(const vbq_gemm_plan *P /* host */, int M, size_t *bytes /* host */);

/*
 * Y = X W^T for M tokens (1 <= M <= 2^20; meant for M > 16, where the
 * product is a dense contraction) from a GEMM plan: x fp16 [M][ldx] (ldx >= K,
 * ldx % 8 == 0, x 16-byte aligned), y [M][ldy] (ldy >= N) in yt.  Each weight
 * enters the matrix cores as fp16(s * (q - (2^b-1)/2)) (one rounding to
 * nearest even), products accumulate in fp32, so
 * |y - y_exact| <= 1e-3 * sum_k |w_k||x_k| + 2^-24 * sum_k |x_k| per output
 * (the second term is the fp16 subnormal spacing; weights at or beyond the
 * fp16 range give non-finite outputs).  The result does not depend on timing.
 * ws: device, 256-byte aligned, >= vbq_gemm_workspace(P, M) bytes, any
 * contents (it holds a copy of X and, where the rows alone do not fill the
 * device, partial sums of K-splits); calls sharing a workspace must be
 * ordered (one stream).  Two launches.  Errors: VBQ_ERR_INVALID_ARG,
 * VBQ_ERR_LAYOUT, VBQ_ERR_BATCH, VBQ_ERR_SHAPE, VBQ_ERR_ALIGN,
 * VBQ_ERR_WORKSPACE.
 */
vbq_status vbq_gemm(const vbq_gemm_plan *P /* host */, const void *buf, int M, const uint16_t *x, int ldx, void *y,
                    int ldy, vbq_dtype yt, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dense fp16 control at the same shapes: y[M][ldy] = W16 x with W16 fp16
 * [N][K] row-major (typically vbq_dequant(..., VBQ_F16)), fp32 accumulate.
 * K % 8 == 0, 1 <= M <= 16.
 */
vbq_status vbq_dense_f16_gemv(int N, int K, int M, const uint16_t *w16, const uint16_t *x, int ldx, void *y, int ldy,
                              vbq_dtype yt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VBQ_H */
