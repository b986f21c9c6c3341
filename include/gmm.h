/*
 * gmm.h -- C ABI of the MI355X (gfx950) MoE grouped matrix multiply library.
 *
 * A grouped matmul (GMM) multiplies the rows of a token matrix that is
 * sorted by expert by that expert's weights: rows [o_g, o_g + s_g) with
 * o_g = s_0 + ... + s_{g-1} use W[g].  ("MoE 优化的探索：从 MiniMax-01、
 * Comet、FlashMoE 到 DeepSeek-V4", section 3.7.2: one independent GEMM per
 * expert, every tile carries its expert id.)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensors are dense and row-major, in device memory of the current
 *    HIP device, and owned by the caller.  The library allocates nothing and
 *    keeps no state between calls (gmm_fp8_fwd_noalloc aside: it keeps a
 *    small device array per GPU).
 *  - `group_sizes` is a device array of G int32 values, read only on the
 *    device (the host never synchronises).  Contract: every s_g >= 0 and
 *    s_0 + ... + s_{G-1} <= M.  Rows at or past that total are written as
 *    zeros by the calls that produce rows ("实现差距：GMM Kernel（V1 vs V2）",
 *    section 3.6).  Sizes outside the contract never make a kernel read or
 *    write outside the caller's buffers: a negative size is read as 0 and
 *    every group's rows are clipped to [0, M) (results are then those of the
 *    clipped groups, and the call's device status says what was wrong).
 *  - Workspace: every grouped call takes `ws`, a device buffer of at least
 *    gmm_workspace_bytes(op, M, K, N, G) bytes, 16-byte aligned, owned by
 *    the caller, needing no initialisation.  The call writes int32 word 0 of
 *    ws with its device status: 0, or an OR of GMM_DEV_SUM_GT_M and
 *    GMM_DEV_NEGATIVE_SIZE (group_sizes broke the contract).  Read it with
 *    gmm_device_status after the call.  Calls that share a workspace and may
 *    run at the same time race on it (the kernels' results are unaffected;
 *    only the status word is).  A missing or too small workspace is
 *    GMM_ERR_WORKSPACE.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns.
 *  - Inputs must be finite.  A quantisation block whose non-zero abs-max is
 *    below 2^-100 is outside the contract.
 *  - Pointers must be 16-byte aligned.  Sizes are element counts.
 *  - Errors: every argument check runs on the host before anything is
 *    launched; on failure the call returns a non-zero gmm_status and
 *    enqueues nothing.  A launch failure returns GMM_ERR_HIP.
 *    gmm_last_error() returns a message for the calling thread's last
 *    failure.
 */
#ifndef GMM_H_
#define GMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define GMM_API __attribute__((visibility("default")))
#else
#define GMM_API
#endif

typedef enum {
    GMM_OK = 0,
    GMM_ERR_NULL = 1,      /* a required pointer is NULL */
    GMM_ERR_SHAPE = 2,     /* a size is out of range or not a multiple of 128 */
    GMM_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
    GMM_ERR_DTYPE = 4,     /* unsupported dtype for this argument */
    GMM_ERR_WORKSPACE = 5, /* ws is NULL or smaller than gmm_workspace_bytes() */
    GMM_ERR_HIP = 6        /* the HIP runtime reported an error at launch */
} gmm_status;

/* Operations, for gmm_workspace_bytes. */
typedef enum {
    GMM_OP_METADATA = 0,       /* gmm_group_metadata */
    GMM_OP_FP8_FWD = 1,        /* gmm_fp8_fwd */
    GMM_OP_FP8_FWD_SWIGLU = 2, /* gmm_fp8_fwd_swiglu */
    GMM_OP_FP8_MXFP4_FWD = 3,  /* gmm_fp8_mxfp4_fwd */
    GMM_OP_BF16_FWD = 4,       /* gmm_bf16_fwd */
    GMM_OP_TGMM = 5,           /* tgmm_bf16 */
    GMM_OP_DX = 6,             /* gmm_bf16_dx */
    GMM_OP_FP8_INT4_FWD = 7    /* gmm_fp8_int4_fwd */
} gmm_op;

/* Bits of the device status word a grouped call writes into its workspace. */
#define GMM_DEV_SUM_GT_M 1       /* the sizes (negative ones read as 0) sum past M */
#define GMM_DEV_NEGATIVE_SIZE 2  /* some group size is negative */

typedef enum {
    GMM_F32 = 0,           /* IEEE binary32 */
    GMM_BF16 = 1,          /* bfloat16 */
    GMM_E4M3 = 2           /* OCP FP8 E4M3 ("fn"): bias 7, max 448, 0x7F NaN */
} gmm_dtype;

/* Largest expert count accepted by the grouped calls. */
#define GMM_MAX_GROUPS 4096

GMM_API const char *gmm_status_string(int status);
GMM_API const char *gmm_last_error(void);

/*
 * gmm_workspace_bytes -- bytes of workspace the grouped call `op` (a gmm_op)
 *   needs for this shape (today 256 for every op: the status block); 0 for
 *   an unknown op.  Sizes are not checked here.
 */
GMM_API size_t gmm_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int64_t G);

/*
 * Tile configurations, for tile searches ("GEMM Kernel 性能优化十问", Q4: the
 * forward, the dX pass and tgmm reduce over different dimensions and get
 * tilings of their own; Q8: the tiling is found by searching).  In an
 * override a 0 field means "the library's choice"; gmm_get_tile_config
 * returns a resolved configuration (the fields the call uses set).
 *   FP8 forwards (GMM_OP_FP8_FWD, _SWIGLU, _MXFP4_FWD, _INT4_FWD; the int4
 *   forward: warp-specialised only, tile_n 512/256/128):
 *     kernel    1 warp-specialised (48 x 512 tiles: 8, 12 or 16 waves, MXFP4:
 *                 16 waves of tile_n 128/256/512 columns), 2 uniform (tile_m
 *                 48/64 rows, tile_n 128/256/512 columns; the only kernel of
 *                 the fused gate+up forward, 256 columns), 3 row-resident
 *                 sweep (one workgroup per 48-row item over all column
 *                 tiles of tile_n 512 for K <= 1024, or of 256, bf16 output,
 *                 for K <= 2048).
 *     waves     warp-specialised: 8 (the one form that also writes the LHS
 *                 codes), 12 or 16.
 *     depth     warp-specialised, 12 waves: K steps of weights in flight, 1 or 2.
 *   bf16 calls (GMM_OP_BF16_FWD, _TGMM, _DX):
 *     kernel    1 128 x 128 tiles, operands staged through registers;
 *                 2 256 x 256 tiles (8 waves, one workgroup per CU; the
 *                 tiled dimensions multiples of 256; forward / dX rows
 *                 from each group's first row); 3 tiles fed by
 *                 load-to-LDS into a ring of LDS stages, 64 x 64 per wave
 *                 (the library's choice for every bf16 call it can take).
 *     waves     kernel 3: 4 (128 x 128 tiles) or 8 (256 x 128, or 128 x 256
 *                 with tile_n 256; tgmm's 256 rows are K rows and need K a
 *                 multiple of 256, the 256 columns a multiple of 256 tiled
 *                 columns).
 *     tile_n    kernel 3 with 8 waves: 128 or 256 (see waves).
 *     depth     kernel 3: LDS stages, 2, 3 or 4 (slices in flight = depth -
 *                 1; slices 64 deep when the rings of all resident
 *                 workgroups fit the LDS, else 32).
 *     residency workgroups per CU the register allocation allows.  Kernel 1:
 *                 2 or 3; kernel 2: 1; kernel 3 with 4 waves: 2 with depth
 *                 2, 1-3 with depth 3, 1-2 with depth 4; with 8 waves:
 *                 depth 3 and residency 2.
 *     placement tgmm: 1 (each XCD takes whole groups) or 2 (every group
 *                 spread over the 8 XCDs, groups in decreasing size class;
 *                 needs a multiple of 8 tiles per group); left 0, each
 *                 call decides from the group sizes (2 when the largest
 *                 group holds more than four times the mean rows).  Forward
 *                 and dX: 1 (row tiles aligned to absolute rows) or 2
 *                 (tiles starting at each group's first row: no tile
 *                 straddles two groups); the library takes 2 for dX and
 *                 for large forward grids.
 */
typedef struct {
    int32_t kernel, waves, tile_m, tile_n, depth, residency, placement;
} gmm_tile_config;

/*
 * gmm_set_tile_config -- replace the library's tile choice for one
 *   operation (a gmm_op with a configuration, not GMM_OP_METADATA),
 *   process-wide, until the next call; cfg NULL restores the library's
 *   choice.  Field values out of range are GMM_ERR_SHAPE here; a
 *   configuration that does not fit a later call's shape makes that call
 *   return GMM_ERR_SHAPE (with the reason in gmm_last_error).  Not for use
 *   while other threads call the library.
 */
GMM_API int gmm_set_tile_config(int op, const gmm_tile_config *cfg);

/*
 * gmm_get_tile_config -- the configuration a call of op on this shape would
 *   run (lhs_dtype and out_dtype as for that call), override included.
 */
GMM_API int gmm_get_tile_config(int op, int64_t M, int64_t K, int64_t N, int64_t G,
                                int lhs_dtype, int out_dtype, gmm_tile_config *cfg);

/*
 * gmm_probe_stream_read -- a platform probe, not part of the grouped
 *   matmul: reads `bytes` of buf with one 64 KB slice per workgroup and
 *   16-byte loads, so that the caller can time the streaming rate this part
 *   delivers from its caches and from HBM ("GEMM Kernel 性能优化十问", Q10,
 *   step 0: measure the platform's bandwidth first).  bytes: a positive
 *   multiple of 65536.  sink: bytes/65536 uint32 words (written only in the
 *   unlikely case that a slice's words XOR to 0x9e3779b9).
 */
GMM_API int gmm_probe_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/*
 * gmm_device_status -- the device status word the last grouped call wrote
 *   into ws (0 = group_sizes kept the contract; else GMM_DEV_* bits), copied
 *   to *status once the work queued on `stream` before it has finished.
 *   Unlike every other call this one synchronises the host with the stream.
 */
GMM_API int gmm_device_status(const void *ws, int32_t *status, void *stream);

/*
 * gmm_group_metadata -- the device-side work list every grouped kernel
 * builds in its prologue, written out for inspection.
 *   Row tiles of height tile_m are aligned to absolute row indices.  For
 *   every non-empty group g (in order) and every tile t that intersects its
 *   rows, one entry {g, t, row_lo, row_hi} with row_lo = max(o_g, t*tile_m)
 *   and row_hi = min(o_g + s_g, (t+1)*tile_m); then one entry {G, t, lo, hi}
 *   per tile holding rows at or past the total (the rows to zero).
 *   ("GEMM Kernel 性能优化十问", Q7 names group indexing among the GMM's
 *   costs; "实现差距：GMM Kernel（V1 vs V2）", gap table: the metadata is
 *   filled inside the kernel.)
 * offsets:  device int32 [G+1], exclusive prefix sums of group_sizes.
 * work:     device int32 [capacity][4].
 * num_work: device int32 [1], number of entries written.
 * Group rows are the clipped ranges of the conventions above; offsets hold
 * their first rows, clipped to M, and offsets[G] the clipped total.
 * capacity must be >= ceil(M/tile_m) + G + 1; tile_m a multiple of 16 in
 * [16, 1024].  ws: as for every grouped call (GMM_OP_METADATA).
 */
GMM_API int gmm_group_metadata(const int32_t *group_sizes, int64_t G, int64_t M,
                       int64_t tile_m, int32_t *offsets, int32_t *work,
                       int64_t capacity, int32_t *num_work, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * gmm_quantize_lhs -- 1x128 dynamic quantisation of the activations.
 *   For every row m and 128-wide block b: a = max |x[m, 128b:128b+128]|,
 *   s = a/448, inv = (s == 0 ? 0 : 1/s), q = e4m3_rne(x * inv), each step
 *   one correctly rounded fp32 operation ("GEMM Kernel 性能优化十问", Q2:
 *   one scale per row per 128 elements; "实现差距：GMM Kernel（V1 vs V2）",
 *   section 3.3: abs-max, scale, guarded inverse, cast).
 * x:     [M,K], x_dtype GMM_BF16 or GMM_F32.
 * q:     [M,K] E4M3 codes.
 * scale: [M,K/128] fp32, the s of each block.
 * K must be a multiple of 128; M >= 1.
 */
GMM_API int gmm_quantize_lhs(const void *x, int x_dtype, int64_t M, int64_t K,
                     uint8_t *q, float *scale, void *stream);

/*
 * gmm_quantize_rhs -- 128x128 block quantisation of the expert weights
 * (done once, offline: "GEMM Kernel 性能优化十问", Q2 and Q5).
 *   Same recipe as gmm_quantize_lhs over each 128x128 block (g, kb, nb).
 * w:     [G,K,N], w_dtype GMM_BF16 or GMM_F32.
 * q:     G*N*K bytes of E4M3 codes in the packed order gmm_fp8_fwd reads
 *        (the MFMA operand layout): [G][N/16][K/128][2][64][16], where byte
 *        (h, l, e) of slab (g, nb, kb) is the code of column n = 16*nb + l%16,
 *        k = 128*kb + 32*(l/16) + 16*h + e.
 * scale: [G,K/128,N/128] fp32.
 * K and N must be multiples of 128.
 */
GMM_API int gmm_quantize_rhs(const void *w, int w_dtype, int64_t G, int64_t K,
                     int64_t N, uint8_t *q, float *scale, void *stream);

/*
 * gmm_pack_rhs -- weights quantised elsewhere into the forward's operand
 *   order: E4M3 codes in the logical [G,K,N] row-major layout (the RHS of
 *   "实现差距：GMM Kernel（V1 vs V2）", section 2.1, whose 128x128 block
 *   scales [G,K/128,N/128] gmm_fp8_fwd takes unchanged) are rewritten in the
 *   packed order gmm_quantize_rhs writes.  A pure permutation: byte (h, l, e)
 *   of slab (g, nb, kb) = q[g, 128*kb + 32*(l/16) + 16*h + e, 16*nb + l%16].
 * q:      [G,K,N] E4M3 codes.     packed: G*N*K bytes, not overlapping q.
 * K and N must be multiples of 128; 1 <= G <= GMM_MAX_GROUPS.
 */
GMM_API int gmm_pack_rhs(const uint8_t *q, int64_t G, int64_t K, int64_t N,
                         uint8_t *packed, void *stream);

/*
 * gmm_quant_scales -- the scale pair of the 1x128 / 128x128 recipe for a
 *   list of block abs-maxima: scale[i] = a/448 and inv[i] = (scale[i] == 0 ?
 *   0 : 1/scale[i]), each correctly rounded fp32, computed by the same device
 *   routines every quantiser of this library and the fused forward use
 *   ("实现差距：GMM Kernel（V1 vs V2）", section 3.3: scale from the abs-max,
 *   guarded inverse).  Exposed so the recipe's arithmetic can be checked on
 *   its own.
 * amax: [n] fp32, each 0 or in [2^-100, FLT_MAX] (the contract's range).
 * scale, inv: [n] fp32.
 */
GMM_API int gmm_quant_scales(const float *amax, int64_t n, float *scale, float *inv,
                             void *stream);

/*
 * gmm_quantize_rhs_mxfp4 -- MXFP4 quantisation of the expert weights (done
 *   once, offline).  "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1:
 *   the RHS may be a sub-byte type, MXFP4 first.  Format and conversion are
 *   the OCP Microscaling (MX) specification v1.0's: each block of 32
 *   consecutive k of one (expert g, column n) shares an E8M0 scale
 *   2^(e-127), e = floor(log2(max |w|)) - 2 clamped to [-127, 127] (code 0
 *   for an all-zero block), and each element is the E2M1 value (0, 0.5, 1,
 *   1.5, 2, 3, 4, 6 and negatives) nearest to w / 2^e, ties to the even
 *   mantissa, clamped to +-6, sign kept.
 * w:     [G,K,N], w_dtype GMM_BF16 or GMM_F32.
 * q:     G*K*N/2 bytes of E2M1 codes in the packed order gmm_fp8_mxfp4_fwd
 *        reads: chunk c = (g*N/16 + n/16)*K/128 + k/128 is 1024 bytes; lane
 *        l = 16*swap2((k%128)/32) + n%16 (swap2 exchanges the two bits of a
 *        2-bit value) owns bytes c*1024 + 16l .. +15, the 32 codes of its
 *        block in k order, two per byte, even k in the low nibble.
 * scale: G*K*N/32 bytes: byte c*64 + l is the E8M0 code of lane l's block.
 * K and N must be multiples of 128.  Errors as for gmm_quantize_rhs.
 */
GMM_API int gmm_quantize_rhs_mxfp4(const void *w, int w_dtype, int64_t G, int64_t K,
                     int64_t N, uint8_t *q, uint8_t *scale, void *stream);

/*
 * gmm_fp8_mxfp4_fwd -- grouped matmul forward of a 1x128 FP8 LHS against
 *   MXFP4 weights.
 *   out[m,n] = sum_b sl[m,b] * sum_{k in 128-block b}
 *                ql[m,k] * e2m1(q4[g,k,n]) * 2^(e8[g,k/32,n] - 127)
 *   for m in group g, accumulated in fp32 (each MFMA sums its 128 products
 *   with a truncation of about 2^-14 of the largest); rows past the
 *   total are 0.  (The forward of gmm_fp8_fwd with the weights in the
 *   sub-byte type of "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1.)
 * lhs, lhs_dtype, lhs_scale: as for gmm_fp8_fwd (bf16/fp32 quantised in the
 *            kernel with the gmm_quantize_lhs recipe, or E4M3 codes + scales).
 * rhs_q, rhs_scale: exactly as written by gmm_quantize_rhs_mxfp4.
 * out:       [M,N], GMM_BF16 or GMM_F32.
 * K and N must be multiples of 128; 1 <= G <= GMM_MAX_GROUPS.
 * Errors: as for gmm_fp8_fwd.
 */
GMM_API int gmm_fp8_mxfp4_fwd(const void *lhs, int lhs_dtype, const float *lhs_scale,
                const uint8_t *rhs_q, const uint8_t *rhs_scale,
                const int32_t *group_sizes, int64_t M, int64_t K, int64_t N,
                int64_t G, void *out, int out_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * gmm_quantize_rhs_int4 -- int4 quantisation of the expert weights (done
 *   once, offline).  "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1
 *   list int4 beside float4_e2m1fn as sub-byte RHS types and give no scale
 *   format; this library keeps the FP8 path's 128x128 blocks and the section
 *   3.3 recipe with the int4 maximum 7: a = max |w| of the block, s = a/7,
 *   inv = (s == 0 ? 0 : 1/s) (each correctly rounded fp32), code =
 *   round-half-even(w * inv) in [-7, 7].
 * w:     [G,K,N], w_dtype GMM_BF16 or GMM_F32.
 * q:     G*K*N/2 bytes of two's-complement int4 codes in the packed order
 *        gmm_fp8_int4_fwd reads: slab c = (g*N/16 + n/16)*K/128 + k/128 is
 *        1024 bytes; lane l = 16*((k%128)/32) + n%16 owns bytes c*1024 + 16l
 *        .. +15 holding rows j = k%32 of its column, byte 4d + i carrying
 *        row j = 8d + i in its low nibble and row 8d + 4 + i in its high one.
 * scale: [G,K/128,N/128] fp32.
 * K and N must be multiples of 128.  Errors as for gmm_quantize_rhs.
 */
GMM_API int gmm_quantize_rhs_int4(const void *w, int w_dtype, int64_t G, int64_t K,
                    int64_t N, uint8_t *q, float *scale, void *stream);

/*
 * gmm_pack_rhs_int4 -- int4 codes made elsewhere, one int8 value in [-8, 7]
 *   per weight in the logical [G,K,N] row-major layout (with [G,K/128,N/128]
 *   fp32 block scales, which gmm_fp8_int4_fwd takes unchanged), rewritten in
 *   the packed order gmm_quantize_rhs_int4 writes.  Values outside [-8, 7]
 *   keep their low 4 bits.
 * q: [G,K,N] int8.  packed: G*K*N/2 bytes, not overlapping q.
 * K and N must be multiples of 128; 1 <= G <= GMM_MAX_GROUPS.
 */
GMM_API int gmm_pack_rhs_int4(const int8_t *q, int64_t G, int64_t K, int64_t N,
                              uint8_t *packed, void *stream);

/*
 * gmm_fp8_int4_fwd -- grouped matmul forward of a 1x128 FP8 LHS against
 *   int4 weights with 128x128 block scales.
 *   out[m,n] = sum_b sl[m,b] * sr[g,b,n/128] * sum_{k in block b} ql[m,k] q4[g,k,n]
 *   for m in group g, accumulated in fp32; rows past the total are 0.  The
 *   forward of gmm_fp8_fwd with the weights in the int4 type of
 *   "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1; the codes are
 *   expanded to E4M3 (exact for every int4 value) in registers.
 * lhs, lhs_dtype, lhs_scale: as for gmm_fp8_fwd.
 * rhs_q:     packed int4 codes (gmm_quantize_rhs_int4 or gmm_pack_rhs_int4).
 * rhs_scale: [G,K/128,N/128] fp32.
 * out:       [M,N], GMM_BF16 or GMM_F32.
 * K and N must be multiples of 128; 1 <= G <= GMM_MAX_GROUPS.
 * ws, ws_bytes: at least gmm_workspace_bytes(GMM_OP_FP8_INT4_FWD, ...).
 * Errors: as for gmm_fp8_fwd.
 */
GMM_API int gmm_fp8_int4_fwd(const void *lhs, int lhs_dtype, const float *lhs_scale,
                const uint8_t *rhs_q, const float *rhs_scale,
                const int32_t *group_sizes, int64_t M, int64_t K, int64_t N,
                int64_t G, void *out, int out_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * gmm_fp8_fwd -- blockwise-FP8 grouped matmul forward.
 *   out[m,n] = sum_b ( sum_{k in block b} ql[m,k] qr[g,k,n] )
 *                    * sl[m,b] * sr[g,b,n/128]        for m in group g,
 *   accumulated in fp32 (each MFMA sums its 128 exact FP8 products with a
 *   truncation of about 2^-14 of the largest); rows past the total are 0.
 *   ("GEMM Kernel 性能优化十问", Q3: each 128-wide K subchannel is scaled and
 *   accumulated separately while the K loop runs over many subchannels;
 *   "实现差距：GMM Kernel（V1 vs V2）", sections 2.1 and 3.3.)
 * lhs:       [M,K].  lhs_dtype GMM_BF16 or GMM_F32: quantised inside the
 *            kernel with the gmm_quantize_lhs recipe (bit-identical codes
 *            and scales); GMM_E4M3: codes, with lhs_scale [M,K/128].
 * lhs_scale: NULL unless lhs_dtype == GMM_E4M3.
 * rhs:       packed E4M3 codes and rhs_scale [G,K/128,N/128] fp32, exactly as
 *            written by gmm_quantize_rhs.
 * out:       [M,N], out_dtype GMM_BF16 (round to nearest even) or GMM_F32.
 * q_out, scale_out: NULL, or [M,K] codes and [M,K/128] scales that receive
 *            the in-kernel quantisation of lhs (only with bf16/f32 lhs).
 *            Only the rows of groups are written; rows at or past the total
 *            are left as they were.
 * K and N must be multiples of 128; 1 <= G <= GMM_MAX_GROUPS.
 */
GMM_API int gmm_fp8_fwd(const void *lhs, int lhs_dtype, const float *lhs_scale,
                const uint8_t *rhs, const float *rhs_scale,
                const int32_t *group_sizes, int64_t M, int64_t K, int64_t N,
                int64_t G, void *out, int out_dtype, uint8_t *q_out,
                float *scale_out, void *ws, size_t ws_bytes, void *stream);

/*
 * gmm_fp8_fwd_noalloc -- gmm_fp8_fwd for callers that cannot allocate device
 *   memory or hand in a workspace: code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc.  Same arguments, checks
 *   and results as gmm_fp8_fwd without ws/ws_bytes; the call allocates
 *   nothing.  Its workspace is a library-owned device array of 4096 bytes,
 *   one per GPU, held from the first call on that GPU until the process
 *   ends; a shape whose gmm_workspace_bytes(GMM_OP_FP8_FWD, ...) exceeds it
 *   is rejected with GMM_ERR_WORKSPACE.  Every call on one GPU shares that
 *   GPU's array and finds the previous call's contents in it (nothing in it
 *   needs to start at zero): calls that may overlap on one GPU race on it.
 *   The device status word goes to that array and is not reported.
 */
GMM_API int gmm_fp8_fwd_noalloc(const void *lhs, int lhs_dtype, const float *lhs_scale,
                const uint8_t *rhs, const float *rhs_scale,
                const int32_t *group_sizes, int64_t M, int64_t K, int64_t N,
                int64_t G, void *out, int out_dtype, uint8_t *q_out,
                float *scale_out, void *stream);

/*
 * gmm_fp8_fwd_swiglu -- blockwise-FP8 grouped matmul with the gate and up
 *   projections fused into one call and the activation applied in the
 *   kernel ("实现差距：GMM Kernel（V1 vs V2）", sections 3.5 and 4.2: the RHS
 *   concatenates the gate weights (first N columns) and the up weights (next
 *   N columns); the kernel returns silu(gate) * up).
 *   With P = the gmm_fp8_fwd product against the 2N-column RHS:
 *     out[m,j] = silu(P[m,j]) * P[m,N+j],  silu(z) = z / (1 + exp(-z)),
 *   computed in fp32; rows past the total are 0.
 * lhs, lhs_dtype, lhs_scale: as for gmm_fp8_fwd.
 * rhs, rhs_scale: gmm_quantize_rhs output for the [G,K,2N] fused weights.
 * out:       [M,N], GMM_BF16 or GMM_F32.
 * act_q, act_scale: NULL, or [M,N] E4M3 codes and [M,N/128] fp32 scales that
 *            receive the 1x128 quantisation of the fp32 activation (the
 *            gmm_quantize_lhs recipe), ready to be the next layer's LHS.
 *            Rows past the total get code 0 and scale 0.
 * K must be a multiple of 128 and N of 256; 1 <= G <= GMM_MAX_GROUPS.
 * Errors: as for gmm_fp8_fwd; act_q and act_scale must both be set or both
 * NULL (GMM_ERR_NULL).
 */
GMM_API int gmm_fp8_fwd_swiglu(const void *lhs, int lhs_dtype, const float *lhs_scale,
                               const uint8_t *rhs, const float *rhs_scale,
                               const int32_t *group_sizes, int64_t M, int64_t K, int64_t N,
                               int64_t G, void *out, int out_dtype, uint8_t *act_q,
                               float *act_scale, void *ws, size_t ws_bytes, void *stream);

/*
 * gmm_bf16_fwd -- unquantised grouped matmul (the bf16 baseline).
 *   out[m,:] = lhs[m,:] . rhs[g(m)] with fp32 accumulation; rows past the
 *   total are 0.  ("GEMM Kernel 性能优化十问", Q10: the BF16 kernel is the
 *   baseline the FP8 kernel is measured against.)
 * lhs: [M,K] bf16.  rhs: [G,K,N] bf16.  out: [M,N] bf16 or f32.
 * K and N must be multiples of 64 (K) and 128 (N).
 */
GMM_API int gmm_bf16_fwd(const void *lhs, const void *rhs, const int32_t *group_sizes,
                 int64_t M, int64_t K, int64_t N, int64_t G, void *out,
                 int out_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * tgmm_bf16 -- weight gradient of the grouped matmul.
 *   dw[g] = sum over rows m of group g of x[m,:]^T dy[m,:], fp32
 *   accumulation; an empty group gives exactly 0.  The reduction runs over
 *   M, so tiles are chosen separately from the forward pass
 *   ("GEMM Kernel 性能优化十问", Q4; Q5: the backward pass is bf16).
 * x: [M,K] bf16.  dy: [M,N] bf16.  dw: [G,K,N] bf16 or f32.
 * K and N must be multiples of 128.  Rows past the total are ignored.
 */
GMM_API int tgmm_bf16(const void *x, const void *dy, const int32_t *group_sizes,
              int64_t M, int64_t K, int64_t N, int64_t G, void *dw,
              int out_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * gmm_bf16_dx -- input gradient of the grouped matmul.
 *   dx[m,:] = dy[m,:] . w[g(m)]^T (contracting over N), fp32 accumulation;
 *   rows past the total are 0.  ("GEMM Kernel 性能优化十问", Q5.)
 * dy: [M,N] bf16.  w: [G,K,N] bf16 (the forward weights, not transposed).
 * dx: [M,K] bf16 or f32.  K multiple of 128, N multiple of 64.
 */
GMM_API int gmm_bf16_dx(const void *dy, const void *w, const int32_t *group_sizes,
                int64_t M, int64_t K, int64_t N, int64_t G, void *dx,
                int out_dtype, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GMM_H_ */
