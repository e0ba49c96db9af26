/*
 * cpattn -- per-rank attention of ring and Ulysses context parallelism on
 * AMD Instinct MI355X (gfx950).
 *
 * The computation is the one a context-parallel rank runs inside its attention
 * backend: a non-causal, unmasked attention forward of the rank's query shard
 * against a sequence of key/value chunks, each step producing a partial output
 * and its log-sum-exp (LSE), the partials merged in fp32 by LSE rescaling, and
 * the Ulysses sequence<->head regroup as a local permute.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers.  The caller owns all memory;
 *     the library never allocates or frees device memory.  Scratch space is
 *     passed in by the caller (cpattn_ring_fwd's workspace).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it and returns; there is no host<->device
 *     synchronisation anywhere, and `chunk_lens` is read on the host.
 *   - Every argument is validated before anything is launched; on any error
 *     nothing is launched and nothing is written.  The return value is a
 *     cpattn_status; cpattn_last_error() gives a message for the calling
 *     thread's most recent failure.
 *   - Tensors are row-major and contiguous unless a leading dimension is given.
 *     Attention tensors use the [B, H, S, d] layout (sequence dim -2), the layout
 *     the ParaAttention README shards with chunk(world_size, dim=-2).
 *   - LSE values are natural logs of sum_j exp(scale * q.k_j), fp32, [B, H, Sq].
 *     A row that saw no key has LSE = -inf and output 0.
 *   - Calls are thread-safe.  Outputs must not overlap inputs except where an
 *     argument is documented as updated in place.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CPATTN_BF16 = 0, /* bfloat16: attention inputs/outputs; products on the bf16 MFMA, P rounded to bf16 */
    CPATTN_FP32 = 1, /* float32: inputs are rounded to bf16 (nearest-even) when staged for the MFMA path */
    CPATTN_FP16 = 2  /* float16: inputs/outputs; products on the fp16 MFMA, P rounded to fp16 */
} cpattn_dtype;

typedef enum {
    CPATTN_OK = 0,
    CPATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    CPATTN_ERR_SHAPE = 2,       /* a size is out of range (B, H < 1; S < 0; kv_ld < Skv; unsupported d) */
    CPATTN_ERR_DEGREE = 3,      /* ring or Ulysses degree < 1, or Ulysses group out of range */
    CPATTN_ERR_INDIVISIBLE = 4, /* sequence or heads do not divide by the degree (no explicit lengths) */
    CPATTN_ERR_CHUNKS = 5,      /* a chunk length < 0, or the lengths do not sum to Skv */
    CPATTN_ERR_DTYPE = 6,       /* unsupported dtype / element size / direction */
    CPATTN_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required */
    CPATTN_ERR_ALIAS = 8,       /* an output overlaps an input it must not overlap */
    CPATTN_ERR_HIP = 9          /* the HIP runtime reported an error; see cpattn_last_error() */
} cpattn_status;

/*
 * cpattn_block_fwd -- one chunk step: attention of Q against one K/V block.
 *
 * Defines: out = softmax(Q K^T * scale) V and lse = log sum_j exp(scale * q.k_j)
 * per query row -- the ring step in which a rank attends its own queries to the
 * K/V chunk it currently holds (ring_degree in ContextParallelConfig,
 * "Parallelism" API page), with the unmasked, non-causal, dropout-free scaled_dot_product_attention
 * semantics of the ParaAttention README example.
 *
 *   q    [B, H, Sq, d]  in_dtype, contiguous.
 *   k, v planes of Skv rows: plane (b, h) starts at element (b*H + h) * kv_ld * d
 *        of the buffer, rows [0, Skv) are used, rows are d contiguous elements.
 *        kv_ld >= Skv lets a chunk of a larger resident K/V buffer be passed in
 *        place (pointer advanced to the chunk's first row).
 *   q, k, v share in_dtype (CPATTN_BF16, CPATTN_FP16 or CPATTN_FP32).
 *   out  [B, H, Sq, d]  out_dtype (CPATTN_FP32 keeps the partial in fp32, the
 *        convert_to_fp32 ring numerics; CPATTN_BF16 / CPATTN_FP16 round to
 *        nearest-even).  Any in_dtype / out_dtype pair is accepted.
 *   lse  [B, H, Sq]     fp32, natural log.
 *   d    64 or 128.  scale <= 0 (or NaN) selects 1/sqrt(d).
 *   Skv == 0 gives out = 0 and lse = -inf.  Sq == 0 is a no-op.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIAS (out/lse overlapping q/k/v), ERR_HIP.
 */
int cpattn_block_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t kv_ld, int64_t d,
                     float scale, int in_dtype, int out_dtype, void* stream);

/*
 * cpattn_lse_merge -- fold one partial into an fp32 accumulator by LSE rescaling.
 *
 * Defines, per row r (the log-sum-exp identity for attention over two disjoint
 * key sets; fp32 as convert_to_fp32 asks, "Parallelism" API page):
 *   L            = log(exp(acc_lse[r]) + exp(blk_lse[r]))
 *   acc_out[r,:] = exp(acc_lse[r] - L) * acc_out[r,:] + exp(blk_lse[r] - L) * blk_out[r,:]
 *   acc_lse[r]   = L
 * A side with LSE = -inf contributes nothing; two such sides give 0 and -inf.
 *
 *   acc_out [rows, d] fp32, acc_lse [rows] fp32: updated in place.
 *   blk_out [rows, d] blk_dtype (CPATTN_FP32, or CPATTN_BF16 / CPATTN_FP16 for 16-bit partials),
 *   blk_lse [rows] fp32.  rows = B*H*Sq.  d a power of two in [4, 256].
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIAS (blk overlapping acc), ERR_HIP.
 */
int cpattn_lse_merge(float* acc_out, float* acc_lse, const void* blk_out, const float* blk_lse,
                     int64_t rows, int64_t d, int blk_dtype, void* stream);

/*
 * Bytes of workspace that are always enough for cpattn_ring_fwd at these sizes,
 * whatever the chunk lengths.  Up to 128 chunks the step runs in one launch and
 * its workspace holds only the pieces of query tiles cut between workgroups:
 * 2 x S slots of min(256, Sq) rows x d fp32 values, then their LSEs at a 256-byte
 * offset, S = 256 (d = 128) or 512 (d = 64) -- at most 67,633,152 (d = 128) or
 * 68,157,440 (d = 64) bytes, independent of B, H and Skv.  Past 128 chunks the
 * per-chunk fallback needs an fp32 [B, H, Sq, d] accumulator when out_dtype is
 * 16-bit.  A call may need less (nothing when no query tile is cut); it checks
 * what its own launch plan writes.  Returns 0 for invalid sizes as well
 * (cpattn_ring_fwd reports those).
 */
size_t cpattn_ring_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t d, int ring_degree,
                                       int out_dtype);

/*
 * cpattn_ring_fwd -- the ring loop of one rank: Q against every K/V chunk in
 * ring order, each step's (partial out, LSE) merged in fp32 by LSE rescaling.
 *
 * Follows the "Context parallelism" page: Ring Attention (each rank attends to
 * one K/V block per step; after the full loop every rank has seen every token),
 * Ring Anything Attention (any sequence length: blocks are sliced back to their
 * true lengths before attention, so padded keys never enter the softmax) and
 * ContextParallelConfig.convert_to_fp32 (partials and LSE kept in fp32).
 * K and V are resident for the whole sequence, as the all-gather rotate method
 * leaves them; chunk c covers rows [off_c, off_c + len_c), off_c = sum of the
 * earlier lengths.
 *
 *   q    [B, H, Sq, d] in_dtype;  k, v [B, H, Skv, d] in_dtype.
 *   out  [B, H, Sq, d] out_dtype; lse [B, H, Sq] fp32.
 *   ring_degree >= 1 chunks.  chunk_lens: HOST array of ring_degree lengths, or
 *   NULL for ring_degree equal chunks (then Skv % ring_degree must be 0, the
 *   plain Ring Attention requirement).
 *   workspace: device memory of cpattn_ring_fwd_workspace_bytes(...) bytes (or at
 *   least what this call's plan writes; NULL when that is 0), 256-byte aligned.
 *   Its contents are scratch.
 *   d 64 or 128; scale <= 0 selects 1/sqrt(d).
 * The whole ring loop runs in one launch (plus a small merge launch when query
 * tiles are cut between workgroups); each chunk's partial is merged into the
 * fp32 accumulator by LSE rescaling as the chunk ends.  Past 128 chunks the
 * step runs one launch per chunk.  Results are bitwise repeatable.
 * Result equals attention over all Skv keys up to fp32 rounding of the merges.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DEGREE, ERR_INDIVISIBLE, ERR_CHUNKS, ERR_DTYPE,
 *         ERR_WORKSPACE, ERR_ALIAS, ERR_HIP.
 */
int cpattn_ring_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                    int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale,
                    int ring_degree, const int64_t* chunk_lens, void* workspace, size_t workspace_bytes,
                    int in_dtype, int out_dtype, void* stream);

/*
 * cpattn_ring_fwd_noalloc -- cpattn_ring_fwd that allocates nothing and takes
 * no workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The pieces of query tiles cut between workgroups go to a scratch array the
 * library holds at file scope on every GPU it runs on, for the life of the
 * process: cpattn_ring_fwd_noalloc_scratch_bytes() bytes (68,157,440), which
 * cover every shape with up to 128 chunks (the scratch grows with the chip's
 * workgroup slots, not with B, H or the sequence lengths).  Its device address
 * is looked up once per device, on the first call there; the call itself makes
 * no hipMalloc, hipFree or other allocating call.  Nothing in the scratch needs
 * clearing between calls: every value a call reads was written by that call.
 * All calls on one GPU share the one array, so calls that overlap on one GPU
 * (two streams, two threads) race: serialise them.
 *
 * Arguments as cpattn_ring_fwd without the workspace; the device is the one
 * `stream` belongs to (the current device for NULL).  Results are bitwise those
 * of cpattn_ring_fwd on the same inputs.
 * Errors: as cpattn_ring_fwd; ERR_DEGREE also for ring_degree > 128 (one launch
 * per chunk would need an accumulator of the problem's size).
 */
int cpattn_ring_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale,
                            int ring_degree, const int64_t* chunk_lens, int in_dtype, int out_dtype,
                            void* stream);

/* Bytes of the scratch array cpattn_ring_fwd_noalloc holds on each GPU. */
size_t cpattn_ring_fwd_noalloc_scratch_bytes(void);

/*
 * cpattn_ring_fwd_cfg -- cpattn_ring_fwd with ContextParallelConfig's
 * convert_to_fp32 switch ("Parallelism" API page: output and LSE cast to fp32
 * to keep the ring numerically stable; on by default).
 *
 *   convert_to_fp32 != 0: exactly cpattn_ring_fwd (fp32 partials and merges).
 *   convert_to_fp32 == 0: the running output between chunk steps is kept in
 *     out_dtype (`out` itself; each merge reads it, merges in fp32 registers and
 *     rounds back to out_dtype); LSE stays fp32 as the attention step produces
 *     it, one launch per chunk.  No workspace is needed.  With out_dtype
 *     CPATTN_FP32 both keep fp32 partials and agree to fp32 rounding and to the
 *     bf16 rounding of the softmax weights against different exponent bases.
 * Other arguments and errors as cpattn_ring_fwd.
 */
int cpattn_ring_fwd_cfg(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale,
                        int ring_degree, const int64_t* chunk_lens, int convert_to_fp32,
                        void* workspace, size_t workspace_bytes, int in_dtype, int out_dtype, void* stream);

/*
 * cpattn_ulysses_permute -- the local half of the Ulysses all-to-all.
 *
 * "Context parallelism" page, Ulysses Attention: after the regroup a rank holds
 * the whole sequence for its share of the heads; the second regroup hands the
 * results back by token.  S and H must divide by the degree P (that page's requirement).
 *
 *   direction 0 (sequence -> head):
 *     in  [P, B, S_local, H, d]: P sequence shards stacked, shard r holding
 *         tokens [r*S_local, (r+1)*S_local) of all H heads.
 *     out [B, H/P, P*S_local, d] for head group `group`:
 *         out[b, h', r*S_local + s, :] = in[r, b, s, group*H/P + h', :]
 *         group = -1 writes all P groups stacked: [P, B, H/P, P*S_local, d].
 *   direction 1 (head -> sequence): the inverse map; `in` is the head-sharded
 *     tensor, `out` the [P, B, S_local, H, d] tensor, of which only the heads of
 *     the given group(s) are written.
 *   elem_bytes: 1, 2, 4 or 8 (bf16 = 2).  The copy is bit-exact.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DEGREE (degree outside [1, 65535] or group outside [-1, P)),
 *         ERR_INDIVISIBLE (H % P), ERR_DTYPE (elem_bytes or direction), ERR_ALIAS
 *         (out overlapping in), ERR_HIP.
 */
int cpattn_ulysses_permute(const void* in, void* out, int64_t B, int64_t S_local, int64_t H, int64_t d,
                           int degree, int group, int direction, int64_t elem_bytes, void* stream);

/*
 * cpattn_ulysses_anything_permute -- the local half of the Ulysses Anything
 * all-to-all: sequence shards and head groups of any sizes.
 *
 * "Context parallelism" page, Ulysses Anything Attention: plain Ulysses needs
 * the sequence length and the head count to divide by the degree; this
 * variant removes both requirements.  Rank r holds seq_lens[r] consecutive
 * tokens (offset off_r = sum of the earlier lengths) and after the regroup
 * head_lens[g] consecutive heads (offset hoff_g).
 *
 *   direction 0 (sequence -> head):
 *     in  the P shards packed back to back: shard r is [B, seq_lens[r], H, d]
 *         at element B * off_r * H * d.
 *     out [B, head_lens[group], S, d] for head group `group`, S = sum(seq_lens):
 *         out[b, h', off_r + s, :] = shard_r[b, s, hoff_group + h', :]
 *         group = -1 writes every group, group g's block at element B * hoff_g * S * d.
 *   direction 1 (head -> sequence): the inverse map; only the heads of the
 *     given group(s) are written into the packed shards.
 *   seq_lens, head_lens: HOST arrays of `degree` counts >= 0; head_lens sum to H.
 *   degree <= 32; elem_bytes 1, 2, 4 or 8.  The copy is bit-exact.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DEGREE (degree outside [1, 32] or group outside
 *         [-1, P)), ERR_CHUNKS (a negative count, or head counts not summing to H),
 *         ERR_DTYPE, ERR_ALIAS, ERR_HIP.
 */
int cpattn_ulysses_anything_permute(const void* in, void* out, int64_t B, int64_t H, int64_t d, int degree,
                                    const int64_t* seq_lens, const int64_t* head_lens, int group,
                                    int direction, int64_t elem_bytes, void* stream);

/*
 * cpattn_unified_fwd -- one rank's share of Unified attention on a
 * ring_degree x ulysses_degree grid of ranks.
 *
 * "Context parallelism" page, Unified Attention: an all-to-all redistributes
 * heads and tokens, Ring Attention runs on the result, and the all-to-all is
 * reversed; every rank belongs to one Ulysses group and one ring group.  With
 * the grid's dimensions ordered (ring, Ulysses) as in the ParaAttention README
 * example, rank w = ring_rank * ulysses_degree + ulysses_rank; its Ulysses
 * group is the ulysses_degree ranks sharing its ring_rank (consecutive
 * sequence shards) and its ring group the ring_degree ranks sharing its
 * ulysses_rank.  This call computes, for rank (ring_rank, ulysses_rank):
 *   1. the Ulysses regroup of q inside its Ulysses group -> every token of
 *      segment ring_rank (U * S_local tokens) for head group ulysses_rank, and
 *      of k and v in every Ulysses group -> every token of the grid for that
 *      head group, segments in the rank's ring order (its own first);
 *   2. the ring loop over the ring_degree segments (cpattn_ring_fwd numerics).
 * The reverse regroup that returns outputs by token is cpattn_ulysses_permute
 * (direction 1) over the U outputs of a Ulysses group.
 *
 *   q, k, v  [W, B, S_local, H, d] in_dtype, W = ring_degree * ulysses_degree:
 *            the sequence shards of every rank stacked (shard w holds tokens
 *            [w * S_local, (w + 1) * S_local)), as the all-to-all consumes them.
 *   out  [B, H / U, U * S_local, d] out_dtype;  lse [B, H / U, U * S_local] fp32.
 *   workspace: cpattn_unified_fwd_workspace_bytes(...) bytes, 256-byte aligned:
 *            the regrouped q, k, v and the ring's fp32 accumulator (scratch).
 *   H % ulysses_degree == 0; d 64 or 128; scale <= 0 selects 1/sqrt(d).
 * Errors: ERR_NULL, ERR_SHAPE, ERR_DEGREE (a degree < 1, their product > 65535,
 *         or a rank outside the grid), ERR_INDIVISIBLE, ERR_DTYPE, ERR_WORKSPACE,
 *         ERR_ALIAS, ERR_HIP.
 */
int cpattn_unified_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int64_t B, int64_t S_local, int64_t H, int64_t d, float scale,
                       int ring_degree, int ulysses_degree, int ring_rank, int ulysses_rank,
                       void* workspace, size_t workspace_bytes, int in_dtype, int out_dtype, void* stream);

/* Bytes of workspace cpattn_unified_fwd needs for these sizes (0 for invalid sizes). */
size_t cpattn_unified_fwd_workspace_bytes(int64_t B, int64_t S_local, int64_t H, int64_t d,
                                          int ring_degree, int ulysses_degree, int in_dtype, int out_dtype);

/* Static text for a status code (never NULL). */
const char* cpattn_status_string(int status);

/* Message for the calling thread's most recent failing call ("" if none). */
const char* cpattn_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int cpattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
