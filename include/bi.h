/*
 * bi.h -- C ABI of the batch-invariant reduction library for AMD MI355X (gfx950).
 *
 * Every product entry point computes each output row with a reduction tree
 * fixed by the reduction dimension alone (K for the matmuls, H for RMSNorm,
 * the key position for attention).  Row i therefore returns the same bits
 * whether it is evaluated alone, inside a larger batch, at any position of the
 * batch, or inside a speculative-verification block.  There is no runtime
 * switch for this: invariance is unconditional.
 *
 * Sources (page title, section):
 *   - "Fix/speculative shape invariance" -- Problem: a single row and a short
 *     matrix must not select different matmul paths, and two-pass SDPA must
 *     not derive its split count from the query length; Changes: the canonical
 *     per-row reduction and the single-query split configuration.
 *   - "Batch-invariant kernels: why temperature-0 decoding is still
 *     nondeterministic" -- Mental model (batch invariance; data-parallel vs
 *     split reductions), Case 6 (RMSNorm data-parallel always; matmul one
 *     configuration with no split-K; attention with a fixed split size and
 *     the KV cache updated before the kernel), The boring rule.
 *   - "Fix fp quantized matmul corruption when the quantized dim is not a
 *     multiple of 32" -- Problem and Fix (nvfp4 group size 16 makes
 *     K % 32 == 16 legal; tails must be bounded on loads and stores), Why fix
 *     the kernel rather than reject the dimension.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless stated.  Tensors are dense
 *     row-major.  Every pointer must be aligned to its element size
 *     (BI_ERR_ALIGN otherwise); attention, embedding and the rotary/cache
 *     write also need 16-byte aligned base pointers.  The matmuls and RMSNorm
 *     use 16-byte vector loads when the pointers and row lengths allow it and
 *     element loads otherwise -- with the same reduction tree either way.
 *   - bf16 / f16 data are 16-bit IEEE-style patterns (bfloat16, binary16);
 *     f32 is binary32.  Accumulation is fp32; outputs are rounded to the
 *     output type with round-to-nearest-even.
 *   - The caller owns and allocates every buffer (outputs and workspaces).
 *     The library never allocates, frees or synchronizes; it keeps no mutable
 *     global state.  Calls are asynchronous and ordered on `stream`.
 *   - Inputs are never written.  Outputs are fully overwritten for every
 *     in-range element; no byte outside an output's extent is written.
 *   - Errors: arguments are validated on the host before anything is
 *     launched; on any error nothing is launched and nothing is written.  A
 *     launch failure reported by the runtime returns BI_ERR_LAUNCH.  Every
 *     shape that passes validation is computed correctly -- tails are bounded
 *     on loads and stores, never silently truncated.
 *   - No exception crosses this interface.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BI_OK = 0,
    BI_ERR_NULL = 1,        /* a required pointer is NULL */
    BI_ERR_SHAPE = 2,       /* a dimension is out of range or inconsistent */
    BI_ERR_DTYPE = 3,       /* unsupported data type code */
    BI_ERR_GROUP = 4,       /* illegal quantization mode / group size / bits for the shape */
    BI_ERR_ALIGN = 5,       /* a base pointer is not 16-byte aligned */
    BI_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the *_workspace_bytes figure */
    BI_ERR_LAUNCH = 7,      /* the HIP runtime rejected a launch */
    BI_ERR_UNSUPPORTED = 8  /* legal request this build does not implement */
} bi_status;

typedef enum { BI_BF16 = 0, BI_F16 = 1, BI_F32 = 2 } bi_dtype;
/* Weight layouts of the dense entry points (their w_layout argument). */
typedef enum { BI_W_NATURAL = 0, BI_W_TRANSPOSED = 1, BI_W_PACKED = 2 } bi_wlayout;
typedef enum { BI_AFFINE = 0, BI_NVFP4 = 1, BI_MXFP4 = 2, BI_MXFP8 = 3 } bi_qmode;

/* ------------------------------------------------------------------------
 * Dense matmul   y[m,n] = sum_k x[m,k] * W[n,k]
 * Source: "Fix/speculative shape invariance", Problem and Changes (dense
 * matmul reduced the same way for one row or a short block, for both
 * orientations of the weight); "Batch-invariant kernels ...", Case 3 and
 * Case 6 (one tile configuration for every batch size, no split-K).
 *   x : [M,K] of `dtype`.
 *   w : by w_layout: BI_W_TRANSPOSED [N,K]; BI_W_NATURAL [K,N]; BI_W_PACKED
 *       the tile-packed form of [N,K] written by bi_pack_weights (16-bit
 *       dtypes, K % 128 == 0, x and w 16-byte aligned; BI_ERR_DTYPE,
 *       BI_ERR_SHAPE, BI_ERR_ALIGN otherwise).  Any other w_layout value:
 *       BI_ERR_SHAPE.
 *   y : [M,N] of `dtype` (fp32 accumulation, RNE to `dtype`).
 *   dtype: BI_BF16, BI_F16 or BI_F32.
 *   M >= 1, N >= 1, K >= 1.
 * Row m of y depends only on row m of x, on W and on K -- not on M, N, the
 * weight layout, or where row m sits in x.
 * ------------------------------------------------------------------------ */
bi_status bi_matmul(const void *x, const void *w, void *y,
                    int64_t M, int64_t N, int64_t K,
                    int32_t dtype, int32_t w_layout, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Tile-packed weights (BI_W_PACKED): a one-time layout change of a [N,K]
 * weight that every dense entry point reads with the same reduction tree,
 * hence the same bits, as [N,K].  For row group r (rows 16r .. 16r + 15, rows
 * >= N stored as zeros), K block b (128 elements) and step s (32 of them),
 * 64 x 8 elements are contiguous, lane l = 16 g + c holding
 * W[16r + c][128 b + 32 s + 8 g + e], e = 0..7, at element offset
 * (((r * (K / 128) + b) * 4 + s) * 64 + l) * 8.  The 4 KiB a wave multiplies
 * per block are one piece of memory instead of sixteen 256-byte pieces of
 * sixteen rows, which streams the weight with fewer DRAM pages opened.  Same
 * source as bi_matmul (the layout is free: only the tree is frozen).
 *   bi_packed_weight_bytes: ceil(N / 16) * 16 * K * 2, or 0 when the shape or
 *     dtype cannot be packed (K % 128 != 0, dtype not BI_BF16 / BI_F16).
 *   bi_pack_weights: w [N,K] -> wp (that many bytes), both 16-byte aligned,
 *     stream-ordered; the caller owns both buffers.  Errors: BI_ERR_NULL,
 *     BI_ERR_DTYPE, BI_ERR_SHAPE, BI_ERR_ALIGN.
 * ------------------------------------------------------------------------ */
size_t bi_packed_weight_bytes(int64_t N, int64_t K, int32_t dtype);
bi_status bi_pack_weights(const void *w, void *wp, int64_t N, int64_t K, int32_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dense matmul with a caller workspace: bitwise the same y as bi_matmul.
 * Same source as bi_matmul.  The reduction tree of every output is bi_matmul's
 * (K blocks of 128 in eight slots, block b in slot b mod 8, each slot summed
 * in ascending block order, the slots added pairwise).  For 16 < M <= 64 with
 * transposed 16-bit weights, K a multiple of 128 and 16-byte aligned x, w and
 * workspace, the slots of one output may be computed by different workgroups;
 * the partial sums of aligned slot groups meet in the workspace and are added
 * in the fixed tree order by whichever workgroup finishes last (also for
 * 8 < M <= 16 when N >= 16384, and 12 < M <= 16 when N K > 4096 * 4096; and
 * for 64 < M <= 128 when N < 20480, each 64-row chunk with its own counters
 * and sums -- a verify block on a narrow projection).  Every other call runs
 * bi_matmul's kernels.  w and w_layout as in bi_matmul (the slot
 * form takes BI_W_TRANSPOSED and BI_W_PACKED weights).
 *   ws, ws_bytes: device memory of at least
 *     bi_matmul_ws_workspace_bytes(M, N, K, dtype, w_layout) bytes
 *     (0 means no workspace is needed and ws may be NULL), 16-byte aligned,
 *     filled with zero bytes before its first use.  Its first 64 KiB hold
 *     per-(column tile, row chunk) counters that every call leaves at zero
 *     again, so one workspace sized for the largest shape serves calls of any
 *     shape (the size grows with the rows past 64).
 *     Calls that share a workspace must be ordered (same stream or
 *     synchronised); concurrent ones race.
 *   Errors: as bi_matmul, plus BI_ERR_WORKSPACE when ws is NULL or too small
 *   and BI_ERR_ALIGN when ws is misaligned.
 * ------------------------------------------------------------------------ */
size_t bi_matmul_ws_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t w_layout);
bi_status bi_matmul_ws(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                       int32_t dtype, int32_t w_layout, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gate/up projection fused with the SwiGLU activation of a Llama-style MLP:
 *   a[m, i] = RNE(silu(g) * u),  g = (x . Wg^T)[m, i] and u = (x . Wu^T)[m, i]
 *   each rounded to bf16 first, silu(g) = g / (1 + exp(-g)) in fp32
 * -- bitwise what bi_matmul (or bi_matmul_ws) followed by bi_silu_mul gives.
 * Source: "Batch-invariant kernels ...", Mental model (pointwise ops are
 * invariant, so fusing the activation into the reduction that produces its
 * input changes no tree) and Case 6 (the decoder's MLP).
 *   x    : [M, K] bf16.
 *   w_il : [2F, K] bf16, the gate and up weights interleaved in blocks of 8
 *          rows: rows [16 i, 16 i + 8) are gate rows [8 i, 8 i + 8),
 *          rows [16 i + 8, 16 i + 16) are up rows [8 i, 8 i + 8); as such
 *          (w_layout BI_W_TRANSPOSED) or tile-packed by bi_pack_weights
 *          (BI_W_PACKED).  BI_W_NATURAL: BI_ERR_UNSUPPORTED.
 *   a    : [M, F] bf16, 16-byte aligned.  F % 8 == 0 (BI_ERR_SHAPE otherwise).
 *   ws   : at least bi_matmul_swiglu_workspace_bytes(M, F, K, dtype) bytes,
 *          16-byte aligned, zero-filled before first use.  Its first 64 KiB
 *          are counters that every call leaves zero (as in bi_matmul_ws, and
 *          one workspace may serve both entry points in stream order); the
 *          rest is scratch: the slot form's group sums, or for any other
 *          shape the [M, 2F] gate/up product before the activation.
 *   dtype: BI_BF16 only (BI_ERR_DTYPE otherwise).
 * ------------------------------------------------------------------------ */
size_t bi_matmul_swiglu_workspace_bytes(int64_t M, int64_t F, int64_t K, int32_t dtype);
bi_status bi_matmul_swiglu(const void *x, const void *w_il, void *a, int64_t M, int64_t F, int64_t K,
                           int32_t dtype, int32_t w_layout, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Group-quantized matmul   y = x @ dequantize(W)^T
 * Source: "Fix fp quantized matmul corruption when the quantized dim is not a
 * multiple of 32", Problem (reference x @ dequantize(w).T; nvfp4 group size
 * 16), Fix (bounded K remainder and N tail; loader masks; mxfp4 and mxfp8 at
 * group size 32), Validation (the differential campaign over affine codes of
 * 2 to 8 bits at group sizes 32/64/128, mxfp4, mxfp8 and nvfp4); "Fix/
 * speculative shape invariance", Problem (quantized matmul selected different
 * paths by M).
 *   x      : [M,K] binary16.
 *   y      : [M,N] binary16.
 *   w_layout BI_W_TRANSPOSED (1), quantized along K:
 *     wq [N, K*bits/32] uint32, scales [N, K/gs], biases [N, K/gs].
 *   w_layout BI_W_NATURAL (0), quantized along N:
 *     wq [K, N*bits/32] uint32, scales [K, N/gs], biases [K, N/gs].
 *   w_layout BI_W_PACKED (2): wq is the buffer bi_pack_qweights wrote from
 *     transposed weights (K % 128 == 0, 16-byte aligned; BI_ERR_SHAPE /
 *     BI_ERR_ALIGN otherwise); scales and biases are not read (may be NULL).
 *     Same bits as the transposed call.  Other w_layout values: BI_ERR_SHAPE.
 *   Packing: each stored row is a little-endian bit stream of `bits`-bit
 *   codes: code j in bits [j*bits, (j+1)*bits) of the stream, stream bit i in
 *   bit i % 32 of uint32 word i / 32.  At 4 bits: eight codes per word, the
 *   lowest index along the quantized axis in bits 0..3; at 8 bits: the row's
 *   bytes in order.
 *   qmode BI_AFFINE: bits in 2..8, gs in {32, 64, 128}; binary16 scales s and
 *     biases b; w = s*q + b (q in 0..2^bits-1), evaluated in fp32 (s*q is
 *     exact) and rounded to binary16.
 *   qmode BI_NVFP4: bits 4, gs == 16; codes are e2m1 (sign in bit 3), scales
 *     are one OCP e4m3fn byte per group; w = e2m1(q) * e4m3(s) (exact in
 *     binary16); biases must be NULL.
 *   qmode BI_MXFP4: bits 4, gs == 32; e2m1 codes, scales one OCP MX e8m0 byte
 *     per group (2^(e - 127), 0xFF = NaN); w = binary16(e2m1(q) * 2^(e - 127)),
 *     the exact fp32 product rounded once (RNE; beyond the binary16 range it
 *     is +-inf); biases must be NULL.
 *   qmode BI_MXFP8: bits 8, gs == 32; codes are OCP e4m3fn bytes (S.1111.111
 *     = NaN), scales one e8m0 byte per group; w = binary16(e4m3(q) *
 *     2^(e - 127)), rounded once as for mxfp4; biases must be NULL.
 *   (The pages name the formats and group sizes; the element and scale
 *   encodings are the OCP microscaling specification's.)
 *   Other (qmode, bits, gs) combinations: BI_ERR_GROUP.  The quantized
 *   dimension must be a multiple of gs (BI_ERR_GROUP otherwise).  Any M >= 1
 *   is legal, as is K % 32 == 16 at gs 16, any K in the natural layout and
 *   N % 32 != 0 in the transposed one -- tails are bounded on loads and
 *   stores.  Every mode runs the same K tree.
 * ------------------------------------------------------------------------ */
bi_status bi_qmatmul(const void *x, const uint32_t *wq, const void *scales, const void *biases,
                     void *y, int64_t M, int64_t N, int64_t K,
                     int32_t qmode, int32_t bits, int32_t group_size, int32_t w_layout,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Expert ("gather") quantized matmul of a mixture-of-experts layer:
 *   y[m, :] = x[lhs[m], :] @ dequantize(W[rhs[m]])^T
 * Source: "Fix fp quantized matmul corruption when the quantized dim is not a
 * multiple of 32", The three defects (the tiled gather shares the quantized
 * matmul's K loop and loader, so the sorted and unsorted MoE paths must bound
 * the K remainder and the column tail the same way) and Validation (sorted
 * gather at T = 64, K = 1040; unsorted gather at M = 50, K = 1040).
 * Every row is reduced exactly as bi_qmatmul reduces a row, so row m has the
 * bits of bi_qmatmul(x[lhs[m]], W[rhs[m]]) -- whatever the other rows, their
 * experts, whether the indices are sorted, or how many rows there are.
 *   x      : [x_rows, K] binary16 (2-byte aligned).
 *   lhs_idx: device int32 [M], the token row of each output row, or NULL for
 *            row m (then x_rows >= M, BI_ERR_SHAPE otherwise).
 *   rhs_idx: device int32 [M], the expert of each output row (any order).
 *   wq, scales, biases: E matrices back to back, each laid out as bi_qmatmul
 *            takes one (w_layout 1 transposed or 0 natural; wq 4-byte
 *            aligned), or w_layout 2: E buffers of bi_pack_qweights back to
 *            back (each bi_packed_qweight_bytes long; K % 128 == 0, wq
 *            16-byte aligned), scales and biases not read (may be NULL).
 *   y      : [M, N] binary16.
 *   Modes and code widths: as bi_qmatmul.  1 <= E <= 1023.  A row whose lhs or rhs index is out
 *   of range (a device-side condition the host cannot check) is written as
 *   binary16 NaN; the other rows are unaffected.  Stream-ordered, no
 *   allocation; errors as bi_qmatmul.
 * ------------------------------------------------------------------------ */
bi_status bi_gather_qmatmul(const void *x, const int32_t *lhs_idx, const int32_t *rhs_idx, const uint32_t *wq,
                            const void *scales, const void *biases, void *y, int64_t M, int64_t x_rows, int64_t N,
                            int64_t K, int64_t E, int32_t qmode, int32_t bits, int32_t group_size, int32_t w_layout,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * Tile-packed quantized weights (BI_W_PACKED for bi_qmatmul), a one-time
 * layout change of transposed weights that bi_qmatmul multiplies with the
 * same tree, hence the same bits.  Same source as bi_qmatmul (the layout is
 * free).  For row group r (rows 16r .. 16r + 15; rows >= N are zeros) and K
 * block b (128 codes): 64 lanes x `bits` words of codes in MFMA lane order,
 * lane l = 16g + c holding the `bits` words of row 16r + c for k in
 * [128b + 32g, +32), at word ((r * (K/128) + b) * 64 + l) * bits (at 4 bits:
 * a 1 KiB chunk of four words per lane); after all code chunks, one
 * constants chunk per (r, b) in the same order -- affine: 16 rows x (128/gs)
 * entries scale | bias << 16 (4 bytes each, row-major); nvfp4 / mxfp4 /
 * mxfp8: 16 rows x (128/gs) scale bytes.  A wave reads its codes for a block
 * as one piece and its constants as one small piece.
 *   bi_packed_qweight_bytes: ceil(N/16) * (K/128) * (256 * bits + constants
 *     chunk), or 0 for an illegal mode / group size / bits or K % 128 != 0.
 *   bi_pack_qweights: transposed wq, scales, biases (as bi_qmatmul) -> wqp of
 *     that many bytes; wq and wqp 16-byte aligned.  Stream-ordered; errors as
 *     bi_qmatmul plus BI_ERR_SHAPE when K % 128 != 0.
 * ------------------------------------------------------------------------ */
size_t bi_packed_qweight_bytes(int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size);
bi_status bi_pack_qweights(const uint32_t *wq, const void *scales, const void *biases, void *wqp, int64_t N,
                           int64_t K, int32_t qmode, int32_t bits, int32_t group_size, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RMSNorm   y = (x * inv) * w,   inv = 1 / sqrt(sum_i x_i^2 / H + eps)
 * Source: "Batch-invariant kernels ...", Case 4 (the sum-of-squares tree must
 * not depend on the batch) and Case 6 (data-parallel, one row never split).
 *   x, y : [rows, H] of `dtype`;  w : [H] of `dtype`.
 *   rows >= 1, H >= 1, eps >= 0.
 * ------------------------------------------------------------------------ */
bi_status bi_rmsnorm(const void *x, const void *w, void *y, int64_t rows, int64_t H,
                     float eps, int32_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Residual add fused with the RMSNorm that follows it in a pre-norm block:
 *   x_out = RNE(x + r)          (the bits bi_add gives)
 *   y     = bi_rmsnorm(x_out)   (the same tree, the same bits)
 * Source: as bi_rmsnorm; "Batch-invariant kernels ...", Mental model
 * (pointwise ops are invariant by construction, so fusing the add changes no
 * reduction).
 *   x, r, x_out, y : [rows, H] of `dtype`;  w : [H].  x_out may alias x
 *   (in-place residual); y must not alias x, r or x_out.
 *   Errors: as bi_rmsnorm (BI_ERR_NULL also for r or x_out).
 * ------------------------------------------------------------------------ */
bi_status bi_add_rmsnorm(const void *x, const void *r, void *x_out, const void *w, void *y,
                         int64_t rows, int64_t H, float eps, int32_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Embedding lookup fused with the RMSNorm that reads it (a decoder step's
 * first norm):
 *   x_out[t, :] = table[ids[t], :]   (the bits bi_embed gives: a zero row for
 *                                     an id outside [0, V))
 *   y           = bi_rmsnorm(x_out)  (the same tree, the same bits)
 * Source: as bi_rmsnorm; "Batch-invariant kernels ...", Mental model (a
 * gather is pointwise over rows, so fusing it changes no reduction).
 *   ids : device int32 [T];  table : [V, H] of `dtype` (BI_BF16 or BI_F16);
 *   x_out, y : [T, H];  w : [H].  x_out and y must not alias the table.
 *   One launch when H is a multiple of 8, H <= 4096 and the table, w, x_out
 *   and y are 16-byte aligned; otherwise bi_embed then bi_rmsnorm (and their
 *   requirements).  Errors: as bi_rmsnorm, BI_ERR_DTYPE for BI_F32,
 *   BI_ERR_SHAPE for V outside [1, 2^31).
 * ------------------------------------------------------------------------ */
bi_status bi_embed_rmsnorm(const int32_t *ids, const void *table, void *x_out, const void *w, void *y,
                           int64_t T, int64_t V, int64_t H, float eps, int32_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode / verify / prefill scaled-dot-product attention (GQA).
 * Source: "Fix/speculative shape invariance", Problem and Changes (the
 * softmax reduction layout of a query must be the same alone or inside a
 * short causal block); "Batch-invariant kernels ...", Case 6 (fixed split
 * size with a varying number of splits; cache updated before the kernel).
 *   q, o   : [B, Q, Hq, D] of `dtype` (BI_BF16 or BI_F16).
 *   k, v   : the KV cache of `dtype`, already holding the keys/values of the
 *            Q new tokens: [B, Lcap, Hkv, D] (kv_layout 0) or head-major
 *            [B, Hkv, Lcap, D] (kv_layout 1, where the keys of one head are
 *            contiguous and a chunk is one piece of memory); same bits in
 *            both.  Other kv_layout values: BI_ERR_SHAPE.
 *   kv_len : device int32 [B]; sequence b holds kv_len[b] valid positions.
 *            Query j of sequence b sits at position p = kv_len[b] - Q + j.
 *            With causal != 0 it attends to keys 0..p, else to 0..kv_len[b]-1.
 *            Requires Q <= kv_len[b] <= max_kv_len <= Lcap (not checked on the
 *            host because kv_len lives on the device; positions beyond a
 *            row's limit are never read; a violating value may leave that
 *            sequence's outputs unwritten or wrong, never touches memory
 *            outside the buffers).
 *   Query head h reads key/value head h / (Hq / Hkv); Hq % Hkv == 0.
 *   D must be 128 in this build.  scale is applied to q.k in fp32, in
 *   base-2 units: s = (q.k) * (scale * log2 e) with the constant rounded once
 *   on the host, and every exponential of the softmax is 2^x -- the same
 *   softmax, with exponentials the hardware computes directly.
 *   ws     : device workspace of at least bi_sdpa_workspace_bytes(...) bytes
 *            (the chunk partials), 16-byte aligned; its contents on entry are
 *            ignored.  Calls that share a workspace must be ordered (same
 *            stream or synchronised).
 * Tree (frozen; bi_build_info reports it): keys in chunks of 256 positions,
 * chunks in ranges of 16; a chunk's (max, sum, weighted values) partial, the
 * ranges' partials and the row's result are each added in ascending order.
 * The chunk and range a key falls in depend only on its position, and chunks
 * past a query's last key are never merged, so a row's bits do not depend on
 * B, Q, the other rows or the launch.  Decode and verify shapes take two
 * launches: the chunk partials (in ws), then the range and row levels; with
 * at least two (sequence, KV head) groups per CU of at most 32 query rows
 * over at most 1024 keys, or of at most 48 (query row, 256-key chunk) pairs
 * (one query over 3072 keys, two over 1536), one launch in which a
 * workgroup walks a group's chunks, forms the same partials (in its LDS for
 * groups of at most 8 query rows, else in ws) and runs the range and row
 * levels for the group's rows itself.
 * Prompts -- at least 128 query rows per KV head (Q * Hq / Hkv >= 128) and
 * max_kv_len <= 8192 (at most two ranges) -- take one launch that computes
 * the same tree per block of 128 query rows without partials (ws is then unused, but
 * is still validated, so that a caller's sizing does not depend on the path).
 * ------------------------------------------------------------------------ */
size_t bi_sdpa_workspace_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int32_t Hq, int32_t D);

bi_status bi_sdpa(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                  int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap,
                  int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t causal,
                  int32_t dtype, int32_t kv_layout, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bi_sdpa without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, kernels and bits as bi_sdpa minus ws /
 * ws_bytes: the chunk partials go to a fixed scratch array of
 * bi_sdpa_noalloc_max_bytes() bytes (64 MiB) that the library holds on each
 * GPU it runs on until the process ends.  A shape whose
 * bi_sdpa_workspace_bytes exceeds that returns BI_ERR_WORKSPACE before
 * anything is launched.  Nothing is allocated: the scratch address is looked
 * up (hipGetSymbolAddress) once per device, on the first call made with that
 * device current.  Every call on one GPU shares that GPU's scratch, so calls
 * that overlap in time on one GPU (different streams, no ordering) race;
 * stream-ordered calls are safe.  Errors: as bi_sdpa, plus BI_ERR_LAUNCH if
 * the scratch address cannot be obtained.
 * ------------------------------------------------------------------------ */
size_t bi_sdpa_noalloc_max_bytes(void);
bi_status bi_sdpa_noalloc(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                          int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t causal,
                          int32_t dtype, int32_t kv_layout, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Row log-softmax, token log-probabilities and row mean (the log-prob
 * outputs a sampler and an RL trainer must agree on bit for bit).
 * Source: "Batch-invariant kernels ...", The boring rule (item 1: one
 * reduction strategy at every batch size), The trap (train/serve log-prob
 * mismatch), Sources (the companion library's mean and log-softmax).
 *   x   : [rows, cols] of `dtype` (BI_BF16, BI_F16, BI_F32).
 *   bi_log_softmax  : y fp32 [rows, cols], y = (x - max) - log(sum exp(x - max)).
 *   bi_token_logprob: out fp32 [rows], the same value at column ids[r]
 *                     (ids device int32 [rows]; an id outside [0, cols) gives NaN).
 *   bi_row_mean     : y fp32 [rows], the row sum divided by cols.
 * Tree per row (depends on cols only): 8-element chunks dealt round-robin to
 * 1024 threads, a sequential fold per thread, a xor butterfly per wave, the
 * 16 wave sums in order; the max is exact.  A row's result does not depend
 * on rows or on its position.  Errors: BI_ERR_NULL, BI_ERR_SHAPE (rows or
 * cols < 1), BI_ERR_DTYPE, BI_ERR_ALIGN (x not element-aligned, y / ids not
 * 4-byte aligned).
 * ------------------------------------------------------------------------ */
bi_status bi_log_softmax(const void *x, float *y, int64_t rows, int64_t cols, int32_t dtype, hipStream_t stream);
bi_status bi_token_logprob(const void *x, const int32_t *ids, float *out, int64_t rows, int64_t cols,
                           int32_t dtype, hipStream_t stream);
bi_status bi_row_mean(const void *x, float *y, int64_t rows, int64_t cols, int32_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Pointwise glue of a Llama-style decoder.  Pointwise ops are batch-invariant
 * by construction ("Batch-invariant kernels ...", Mental model).  All tensors
 * are bf16 unless stated.
 * ------------------------------------------------------------------------ */

/* out[t, :] = table[ids[t], :];  ids: device int32 [T] (each in [0, V)),
 * table [V, H], out [T, H].  Ids outside [0, V) produce a zero row. */
bi_status bi_embed(const int32_t *ids, const void *table, void *out, int64_t T, int64_t V,
                   int64_t H, hipStream_t stream);

/* Rotary embedding (rotate-half pairs i, i + D/2) of the q and k parts of a
 * fused projection, then the KV-cache write, in one launch.
 *   qkv   : [B*Q, (Hq + 2*Hkv) * D]; row (b, j) holds q | k | v of token j of
 *           sequence b.
 *   q_out : [B*Q, Hq*D]   rotated q.
 *   kc, vc: caches, [B, Lcap, Hkv, D] (kv_layout 0) or [B, Hkv, Lcap, D]
 *           (kv_layout 1), as bi_sdpa reads them; token j of sequence b is
 *           written at position kv_len[b] - Q + j (rotated k, v unchanged).
 *   cos_t, sin_t: fp32 [max_pos, D/2] tables; positions must be < max_pos.
 *   out_i = x_i * c_i - x_{i+D/2} * s_i;  out_{i+D/2} = x_{i+D/2} * c_i + x_i * s_i
 *   (each product and the difference/sum rounded separately in fp32). */
bi_status bi_rope_kv_write(const void *qkv, void *q_out, void *kc, void *vc,
                           const int32_t *kv_len, const float *cos_t, const float *sin_t,
                           int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                           int32_t D, int64_t max_pos, int32_t kv_layout,
                           hipStream_t stream);

/* out[r, i] = silu(gu[r, i]) * gu[r, F + i],  silu(g) = g / (1 + exp(-g));
 * gu [rows, 2F], out [rows, F]. */
bi_status bi_silu_mul(const void *gu, void *out, int64_t rows, int64_t F, hipStream_t stream);

/* out = a + b (fp32 add, RNE to bf16); n elements; out may alias a or b. */
bi_status bi_add(const void *a, const void *b, void *out, int64_t n, hipStream_t stream);

/* idx[r] = argmax_c x[r, c] over a bf16 [rows, cols] matrix; the lowest
 * index wins ties; idx device int32 [rows]. */
bi_status bi_argmax(const void *x, int32_t *idx, int64_t rows, int64_t cols, hipStream_t stream);

/* Greedy decode step bookkeeping fused into the argmax of its logits (one
 * new token per sequence, rows == sequences): idx[r] = argmax as bi_argmax,
 * ids_next[r] = the same token (the sequence's next input) and kv_len[r] += 1
 * (its cache grows by one position).  ids_next and kv_len: device int32
 * [rows]; kv_len must not be read or written by other work in flight.
 * Errors: as bi_argmax, BI_ERR_NULL for ids_next or kv_len. */
bi_status bi_argmax_advance(const void *x, int32_t *idx, int32_t *ids_next, int32_t *kv_len, int64_t rows,
                            int64_t cols, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Non-invariant comparison variants.  These reproduce the strategies the
 * pages identify as the source of batch dependence -- split-K matmul with a
 * cleanup reduction and an RMSNorm row split across workgroups -- so that
 * the cost of invariance can be measured against the best of them.
 * They are deterministic run to run for fixed arguments, but a caller that
 * picks `splits` from the batch size gets batch-dependent bits.
 * Source: "Batch-invariant kernels ...", Case 2 (split-k), Case 3, Case 4,
 * Case 6 (Split-K / Split-KV); "Fix/speculative shape invariance", Problem.
 * bi_matmul_split takes weights in any layout of bi_matmul.  The quantized
 * and attention variants below are built from the invariant path's own
 * kernels, so that only the tree differs.
 * ------------------------------------------------------------------------ */
size_t bi_matmul_split_workspace_bytes(int64_t M, int64_t N, int32_t splits);
bi_status bi_matmul_split(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                          int32_t dtype, int32_t w_layout, int32_t splits,
                          void *ws, size_t ws_bytes, hipStream_t stream);

size_t bi_rmsnorm_split_workspace_bytes(int64_t rows, int32_t splits);
bi_status bi_rmsnorm_split(const void *x, const void *w, void *y, int64_t rows, int64_t H,
                           float eps, int32_t dtype, int32_t splits,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* Split-K quantized matmul: arguments and result layout of bi_qmatmul, plus
 * `splits` (1 .. K / 128).  Split z reduces the contiguous K blocks
 * [z nb / splits, (z + 1) nb / splits) (nb = K / 128) with the streaming
 * decode kernel's in-block tree, writing fp32 partials [splits, M, N] to ws;
 * a cleanup kernel adds them in z order and rounds to binary16.  splits == 1
 * is bi_qmatmul itself (ws unused).  Takes the 4-bit modes in the transposed
 * (1) or packed (2) layout with M <= 16, K % 128 == 0 and 16-byte aligned x
 * and wq; other shapes: BI_ERR_UNSUPPORTED.  Workspace: at least
 * bi_qmatmul_split_workspace_bytes(M, N, splits) bytes, 16-byte aligned
 * (else BI_ERR_WORKSPACE / BI_ERR_ALIGN).
 * Source: "Fix fp quantized matmul corruption ..." (the quantized decode
 * kernel it is built from); "Batch-invariant kernels ...", Case 2 (split-k). */
size_t bi_qmatmul_split_workspace_bytes(int64_t M, int64_t N, int32_t splits);
bi_status bi_qmatmul_split(const void *x, const uint32_t *wq, const void *scales, const void *biases, void *y,
                           int64_t M, int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size,
                           int32_t w_layout, int32_t splits, void *ws, size_t ws_bytes, hipStream_t stream);

/* Split-KV attention: arguments of bi_sdpa, plus `splits` >= 1.  The chunks
 * of max_kv_len keys (256 each, nch of them) are cut into runs of
 * cps = ceil(nch / min(splits, nch)) chunks; one workgroup walks a run in
 * order with the softmax state carried across its chunks (the chunk tree of
 * bi_sdpa inside each chunk), and the runs' (o, m, l) are merged by
 * bi_sdpa's merge kernel.  A single run writes the output directly (no
 * workspace, one launch).  splits >= nch gives runs of one chunk: bi_sdpa's
 * bits.  Requires Q * (Hq / Hkv) <= 16 (one 16-row query tile per sequence
 * and KV head), else BI_ERR_UNSUPPORTED.  Workspace:
 * bi_sdpa_split_workspace_bytes(B, Q, max_kv_len, Hq, D, splits) bytes (0 for
 * a single run; ws may then be NULL), 16-byte aligned.
 * Source: "Batch-invariant kernels ...", Case 6 (Split-KV: a split count
 * that follows the shape); "Fix/speculative shape invariance", Problem (a
 * split count derived from the query length). */
size_t bi_sdpa_split_workspace_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int32_t Hq, int32_t D,
                                     int32_t splits);
bi_status bi_sdpa_split(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                        int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                        int32_t D, float scale, int32_t causal, int32_t dtype, int32_t kv_layout, int32_t splits,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement hooks (not part of any computation): the next kernel (or the
 * next `count` kernels) that the library's entry points launch from the
 * calling host thread carry `start`, recorded when the first begins
 * executing, and `stop`, recorded when the last ends (hipExtLaunchKernel), so
 * hipEventElapsedTime(start, stop) is their own execution time without the
 * host's launch overhead.  Either event may be NULL; the launches consume the
 * setting (bi_time_next_launches with count 0 clears it; count < 0:
 * BI_ERR_SHAPE).
 * ------------------------------------------------------------------------ */
bi_status bi_time_next_launch(hipEvent_t start, hipEvent_t stop);
bi_status bi_time_next_launches(hipEvent_t start, hipEvent_t stop, int32_t count);

/* ------------------------------------------------------------------------
 * Measurement probes (not part of any computation): the rates this GPU
 * sustains, against which the kernels above are also reported.
 *   bi_probe_read : reads `bytes` (a multiple of 16) from src in 16-byte words
 *                   with `workgroups` workgroups of 256 threads, grid-stride;
 *                   writes 16 bytes per workgroup to sink (workgroups * 16
 *                   bytes).  Bytes moved: `bytes`.
 *   bi_probe_copy : copies `bytes` from src to dst (non-overlapping).  Bytes
 *                   moved: 2 * `bytes`.
 *   bi_probe_mfma : `workgroups` x 4 waves, each issuing iters x 8
 *                   independent v_mfma_f32_16x16x32_bf16 on registers (16384
 *                   flops each); sink: fp32 [workgroups * 256].
 * src, dst and sink 16-byte aligned.  Errors: BI_ERR_NULL, BI_ERR_SHAPE,
 * BI_ERR_ALIGN, BI_ERR_LAUNCH.
 * ------------------------------------------------------------------------ */
bi_status bi_probe_read(const void *src, size_t bytes, void *sink, int32_t workgroups, hipStream_t stream);
bi_status bi_probe_copy(const void *src, void *dst, size_t bytes, int32_t workgroups, hipStream_t stream);
bi_status bi_probe_mfma(void *sink, int32_t workgroups, int64_t iters, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Human-readable status name (static string, never NULL). */
const char *bi_status_str(int32_t status);
/* Static string naming the frozen reduction constants of this build (MFMA
 * instructions, K slicing, attention chunk size, lane mappings). */
const char *bi_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
