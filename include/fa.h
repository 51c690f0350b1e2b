/*
 * fa.h — C ABI of libfa.so: exact tiled attention (FlashAttention) for
 * AMD MI355X (gfx950).
 *
 * Sources (the three web pages on FlashAttention, cited by title + section):
 *   [DEC] "FlashAttention, Decoded: What 'IO-Aware' Actually Means"
 *   [HFL] "FlashAttention: A Novel Attention Algorithm with IO Awareness,
 *          Fast and Memory-Efficient"
 *   [ODP] "FlashAttention: Fast and Memory-Efficient Exact Attention with
 *          IO-Awareness" (opendecode.dev paper page)
 *
 * What every call computes: O = softmax(Q K^T * scale + mask) V, exactly
 * (up to floating-point rounding), without writing the N x N score matrix to
 * device memory ([DEC "Decoding the Abstract", Sentence 4]; [ODP "The key
 * idea"]).  The backward recomputes the score tiles from Q, K and the saved
 * per-row log-sum-exp instead of storing them ([DEC "The Hardware Picture:
 * Why Tiling Wins"], recomputation; [ODP "The key idea"]).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library allocates nothing and frees nothing.  q, k, v, o, dO, dq, dk,
 *   dv are contiguous row-major [B][H][N][d] arrays of the element type
 *   `dtype`, with 16-byte-aligned base addresses.  lse is a contiguous
 *   float32 [B][H][N] array (natural logarithm).  key_len is int32 [B] in
 *   device memory.  block_mask is uint8 [nb][nb] in device memory,
 *   nb = ceil(N / block_size), shared by every (b, h).
 * Sizes.  B >= 1, H >= 1, N >= 1, d in {32, 64, 96, 128}; B*H <= 65535*65535 and
 *   B*H*N*d < 2^31 elements per tensor.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls
 *   only enqueue work on it and return without synchronising.
 * Errors.  Arguments are validated before any HIP call is made:
 *   FA_ERR_INVALID      a null pointer, a size out of range, a non-finite
 *                       or non-positive scale, a workspace that is too small;
 *   FA_ERR_UNSUPPORTED  a valid request the library does not implement
 *                       (d not in {32, 64, 96, 128}, block_size != 128, fp32
 *                       block-sparse);
 *   FA_ERR_HIP          a kernel launch failed (hipGetLastError).  Faults
 *                       during kernel execution surface at the caller's next
 *                       synchronisation, as for any asynchronous launch;
 *   FA_ERR_TOO_LARGE    (fa_bwd_noalloc only) the problem needs more
 *                       workspace than the library's fixed array holds.
 * Masks.  Combined with AND.  causal: key j visible to query i iff j <= i.
 *   key_len (nullable): key j of batch element b visible iff j < key_len[b];
 *   key_len[b] outside [0, N] is clamped to that range.  Rows that see no
 *   key get O = 0, lse = -inf and contribute nothing to the gradients.
 * Thread safety.  Every call is stateless; concurrent calls on different
 *   outputs (and, for the backward and decode, different workspaces) are
 *   safe.  Kernels launch on the calling thread's current HIP device, which
 *   must own `stream` and the tensors.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,
  FA_ERR_UNSUPPORTED = -2,
  FA_ERR_HIP = -3,
  FA_ERR_TOO_LARGE = -4
} fa_status;

/* Element strides of one [B][H][N][d] tensor view: element (b, h, i, c)
 * lies at base + b*batch + h*head + i*row + c (the d index is contiguous).
 * A packed tensor has row = d, head = N*d, batch = H*N*d; the [B][N][H][d]
 * layout of most framework code, viewed as [B][H][N][d], has row = H*d,
 * head = d, batch = N*H*d. */
typedef struct {
  int64_t batch, head, row;
} fa_strides;

/* The strides of every tensor a call touches (fields a call does not use
 * are ignored); a NULL layout means every tensor is packed. */
typedef struct {
  fa_strides q, k, v, o, dO, dq, dk, dv;
} fa_layout;

/* Forward.  [ODP "The key idea"]: the queries, keys and values are split
 * into blocks that fit on-chip, a running row maximum and running row sum
 * are kept per query, and the partial output is rescaled as each key/value
 * tile arrives; [HFL "FlashAttention"]: one fused kernel loads its inputs
 * from HBM once and writes the result once.
 *   q, k, v : inputs [B][H][N][d], dtype
 *   o       : output [B][H][N][d], dtype (same as the inputs)
 *   lse     : output float32 [B][H][N]: scale*max_j s_ij + ln(sum_j exp(...)),
 *             the row statistic the backward reuses; -inf for empty rows
 *   scale   : multiplies Q K^T (usually 1/sqrt(d))
 *   causal  : 0 or 1
 *   key_len : NULL (no padding mask) or int32 [B]
 * dtype FA_F32 computes with fp32 products; FA_F16/FA_BF16 use 16-bit
 * matrix-core products with fp32 accumulation and an fp32 softmax. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* key_len, int dtype, void* stream);

/* Bytes of device workspace fa_bwd / fa_bwd_blocksparse need, about
 * 16*B*H*N + 6*B*H*N*d + 2064*B*H (each region rounded up to 256 bytes):
 * per query row, D_i = sum_c dO_ic O_ic, the base-2 softmax shift
 * lse_i * log2(e) (+inf for rows without keys) and their power-of-two
 * scaled negations (four floats), and 16-bit copies of the row's q, k and
 * dO scaled by powers of two; per (b, h), the maxima of |q|, |k|, |v|,
 * |dO| that choose those powers and the partial maxima of at most 128
 * workgroups of the D pass that they are reduced from.  Linear in N: the method's memory grows
 * linearly, not quadratically, in sequence length ([ODP "Why it
 * mattered"]).  Returns 0 for invalid sizes. */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/* Backward with recomputation ([ODP "The key idea"]; [DEC "The Hardware
 * Picture: Why Tiling Wins"]): the probabilities are rebuilt on-chip from
 * q, k and lse; nothing of size N x N is stored.  Launches on `stream`:
 * D = rowsum(dO * O) with the operand copies; then dK/dV (one workgroup per
 * key tile) and dQ (one workgroup per query tile), for 16-bit inputs as one
 * launch whose grid holds both.  Deterministic: no atomics.
 *   o, lse  : the forward's outputs for the same inputs and mask
 *   dO      : upstream gradient [B][H][N][d], dtype
 *   dq,dk,dv: outputs [B][H][N][d], dtype (overwritten)
 *   workspace / workspace_bytes: device scratch >= fa_bwd_workspace_size
 * dtype FA_F16 or FA_BF16 (16-bit matrix-core products on power-of-two
 * scaled fp16 operands, fp32 accumulation), or FA_F32 (fp32 matrix-core
 * products, P and dS in fp32; the block-sparse form is FA_ERR_UNSUPPORTED
 * for fp32). */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* key_len, void* workspace, size_t workspace_bytes,
           int dtype, void* stream);

/* Block-sparse forward ([DEC "The Passage", block-sparse extension; "Key
 * Vocabulary", block-sparse attention: attention computed only on selected
 * blocks of the score matrix]).  Query i sees key j iff
 * block_mask[i / block_size][j / block_size] != 0.  Unselected blocks are
 * skipped, not masked.  block_size must be 128.  dtype FA_F16 or FA_BF16. */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int H, int N, int d, float scale,
                       const uint8_t* block_mask, int block_size, int dtype,
                       void* stream);

/* Block-sparse backward ([DEC "The Passage", block-sparse extension; "Key
 * Vocabulary", block-sparse attention], with the recomputation of fa_bwd:
 * [ODP "The key idea"]): fa_bwd's gradients of the block-sparse forward,
 * with every tile product restricted to the selected blocks — dK/dV
 * workgroups walk the selected blocks of their key column, dQ workgroups
 * those of their query row; unselected blocks are skipped, never masked.
 *   o, lse    : fa_fwd_blocksparse's outputs for the same inputs and mask
 *   block_mask, block_size: as fa_fwd_blocksparse (block_size must be 128)
 * Other arguments, the workspace and the errors as fa_bwd; dtype FA_F16 or
 * FA_BF16 (FA_F32: FA_ERR_UNSUPPORTED).  Deterministic: no atomics. */
int fa_bwd_blocksparse(const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int B, int H, int N,
                       int d, float scale, const uint8_t* block_mask,
                       int block_size, void* workspace, size_t workspace_bytes,
                       int dtype, void* stream);

/* The stages of fa_bwd / fa_bwd_blocksparse, one at a time, for callers
 * that schedule them separately (to time each kernel, or to place them on
 * different streams with their own events).
 *   stage FA_BWD_STAGE_D    : the workspace: D_i = sum_c dO_ic O_ic, the
 *                             softmax shift, the per-(b, h) maxima and the
 *                             scaled 16-bit copies of q, k and dO
 *                             (two launches; fp32: D and the shift only,
 *                             one launch)
 *   stage FA_BWD_STAGE_DKDV : dk, dv (reads the workspace written by stage 1)
 *   stage FA_BWD_STAGE_DQ   : dq     (reads the workspace written by stage 1)
 *   stage FA_BWD_STAGE_GRADS: dk, dv and dq exactly as fa_bwd launches them
 *                             after stage 1 (16-bit: one launch whose grid
 *                             holds the dK/dV and the dQ workgroups; fp32:
 *                             stages 2 and 3)
 * Running stages 1, 2, 3 in this order on one stream, or stages 1 and 4,
 * gives fa_bwd's results bit for bit: stage 1 followed by stage 4 is
 * exactly the launch sequence of fa_bwd.  The
 * arguments are those of fa_bwd; block_mask non-NULL selects the
 * block-sparse variant (then causal must be 0, key_len NULL and block_size
 * 128; block_size is ignored otherwise).  Pointers a stage does not touch
 * must still be valid arguments.  An unknown stage is FA_ERR_INVALID. */
enum {
  FA_BWD_STAGE_D = 1,
  FA_BWD_STAGE_DKDV = 2,
  FA_BWD_STAGE_DQ = 3,
  FA_BWD_STAGE_GRADS = 4
};
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dO, void* dq,
                 void* dk, void* dv, int B, int H, int N, int d, float scale,
                 int causal, const int32_t* key_len, const uint8_t* block_mask,
                 int block_size, void* workspace, size_t workspace_bytes,
                 int dtype, void* stream);

/* Forward with dropout on the probabilities ([HFL] "Standard Attention
 * Algorithm" names dropout, with masking and softmax, among the elementwise
 * passes that dominate standard attention; here it is fused into the
 * kernel): O = (P * M / (1 - p)) v with M_ij kept iff 16-bit draw t(j) of
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) at counter
 * (g(j), i, b*H + h, offset) and key (seed mod 2^32, seed / 2^32) is >=
 * floor(p 2^16), where g(j) = 2 (j / 16) + (j / 4) mod 2,
 * t(j) = 4 ((j / 8) mod 2) + j mod 4, and draw t is half t mod 2 (low half
 * first) of output word t / 2.  lse is that of P (the un-dropped softmax).  The mask
 * depends only on (seed, offset) and the element's indices, so fa_bwd_dropout
 * regenerates it instead of storing it.  Other arguments as fa_fwd.
 *   dropout_p : in [0, 1); 0 gives fa_fwd's result.  Outside: FA_ERR_INVALID
 * dtype FA_F16 or FA_BF16 (FA_F32 with dropout_p > 0: FA_ERR_UNSUPPORTED). */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_len, float dropout_p, uint64_t seed, uint32_t offset,
                   int dtype, void* stream);

/* Backward of fa_fwd_dropout (same dropout_p, seed, offset, and o, lse from
 * it): dV = (P M')^T dO, dS = P (M' (dO v^T) - D), M' = M / (1 - p).  Other
 * arguments and the workspace as fa_bwd. */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                   int H, int N, int d, float scale, int causal, const int32_t* key_len,
                   float dropout_p, uint64_t seed, uint32_t offset, void* workspace,
                   size_t workspace_bytes, int dtype, void* stream);

/* The forward on tensors of any fa_layout, with every mask and option of
 * the entry points above in one call: causal and key_len (as fa_fwd),
 * block_mask and block_size (as fa_fwd_blocksparse; then causal must be 0,
 * key_len NULL and dropout_p 0), dropout_p, seed and offset (as
 * fa_fwd_dropout; dropout_p = 0: none).  This is the call for tensors that
 * are views of a framework's storage, e.g. [B][N][H][d] activations or the
 * q, k, v slices of a fused projection: the kernels read and write them in
 * place, with no transposing copy ([DEC "The Passage"]: the kernel behind
 * scaled_dot_product_attention, whose inputs are such views).
 *   layout : strides of q, k, v, o in elements (NULL: packed).  Every
 *            stride must be >= 0 and a multiple of 8 elements (16-bit
 *            dtypes) or 4 (FA_F32), row strides below 2^24, and o's row
 *            stride at least d; otherwise FA_ERR_INVALID.  lse is always a
 *            packed [B][H][N] array.
 * Everything else as fa_fwd. */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_len, const uint8_t* block_mask, int block_size,
                   float dropout_p, uint64_t seed, uint32_t offset,
                   const fa_layout* layout, int dtype, void* stream);

/* The backward of fa_fwd_strided (the same mask, dropout and, for q, k, v,
 * o, the same tensors): dq, dk, dv written through their strides in
 * `layout` (row strides at least d); dO read through its strides.  The
 * workspace (fa_bwd_workspace_size) is always packed.  Everything else as
 * fa_bwd. */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_len, const uint8_t* block_mask, int block_size,
                   float dropout_p, uint64_t seed, uint32_t offset,
                   const fa_layout* layout, void* workspace, size_t workspace_bytes,
                   int dtype, void* stream);

/* Bytes of device workspace fa_decode needs: one partial result (d + 2
 * floats) per (b, h, query, key chunk), the keys split into chunks of 256 to
 * 1024 rows.  Linear in Nq and Nk.  Returns 0 for invalid sizes. */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d);

/* Decode: Nq new queries per (b, h) against Nk keys and values (the cached
 * sequence, the new tokens' own keys included), O = softmax(q k^T * scale +
 * mask) v with key j visible to every query iff j < key_len[b] (NULL: all
 * Nk); no causal order among the Nq queries (for Nq = 1 this is causal
 * decoding).  The same exact attention as fa_fwd ([ODP] "The key idea":
 * running maximum and sum, partial outputs rescaled to a common maximum),
 * split over the keys for short query blocks: one launch leaves a partial
 * (O, m, l) per key chunk in the workspace, a second merges them.
 *   q, o    : [B][H][Nq][d], dtype;   k, v: [B][H][Nk][d], dtype
 *   lse     : [B][H][Nq] fp32 (natural log; -inf and O = 0 for a query
 *             without visible keys)
 *   workspace / workspace_bytes: device scratch >= fa_decode_workspace_size
 * dtype FA_F32, FA_F16 or FA_BF16; d 32, 64, 96 or 128.  Products and the softmax
 * run in fp32.  Errors as for fa_fwd (a small workspace is
 * FA_ERR_INVALID). */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int d, float scale, const int32_t* key_len, void* workspace,
              size_t workspace_bytes, int dtype, void* stream);

/* Size in bytes of the device array that fa_bwd_noalloc uses as its
 * workspace (128 MiB; one copy per GPU the library runs on). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* fa_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * It computes exactly what fa_bwd computes (the same kernels and launch
 * sequence), but its workspace is a fixed array of FA_NOALLOC_SCRATCH_BYTES
 * inside the library instead of a caller-provided buffer; it calls no
 * allocation routine.  The caller still passes and owns every input and
 * output.  Dense, causal or key-padded (no block mask, no dropout); dtype
 * FA_F32, FA_F16 or FA_BF16.
 *   Limit: fa_bwd_workspace_size(B, H, N, d) <= FA_NOALLOC_SCRATCH_BYTES,
 *   else FA_ERR_TOO_LARGE (for example B=1, H=16, N=16384, d=64 needs
 *   100 MiB and fits; d=128 at that size needs 196 MiB and does not).
 *   Sharing: every call on one GPU uses that GPU's one array, so calls
 *   that overlap in time on one GPU (different streams or host threads
 *   without ordering between them) race and give wrong results; calls
 *   ordered on one stream are fine.  The array keeps the last call's
 *   contents; nothing in it needs clearing between calls.
 *   Errors: as fa_bwd, checked before any HIP call, plus FA_ERR_TOO_LARGE;
 *   FA_ERR_HIP if the array's device address cannot be obtained (looked up
 *   once per device, on the first call with that device current). */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_len, int dtype, void* stream);

/* Static description of a status code ("ok", "invalid argument", ...). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
