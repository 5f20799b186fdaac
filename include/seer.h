/*
 * seer.h -- C ABI of the MI355X (gfx950) SeerAttention hot path.
 *
 * Pages cited:
 *   [E] "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs"
 *       (paper-graph-ui explainer of arXiv 2410.13276)
 *   [R] "SeerAttention: Self-distilled Attention Gating for Efficient
 *       Long-context Prefilling" (OpenReview discussion, paperhub)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are row-major. Q is [B, Hq, S, D]; K and V are [B, Hkv, S, D]
 *    (grouped-query attention: query head h reads KV head h / (Hq / Hkv)).
 *    Q, K, V are bfloat16 (raw 16-bit patterns, `const void*`).
 *  - Block maps (gate scores, block mask, ground truth) are [B, Hq, nb, nb]
 *    with nb = ceil(S / 64); entry (i, j) is query block i against key block j.
 *    The last block may be ragged (S not a multiple of 64).
 *  - Attention is causal (prefill): key u is visible to query t iff u <= t.
 *    The softmax scale is 1/sqrt(D).
 *  - Every pointer argument except `topk_per_head` is DEVICE memory owned by
 *    the caller. The library allocates nothing, keeps no state between calls
 *    and never synchronizes the host: work is enqueued on `hip_stream`
 *    (a hipStream_t; NULL means the default stream) and outputs are valid
 *    once that stream has reached the end of the call.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    error the call returns a non-zero seer_status, enqueues nothing and
 *    writes nothing; seer_last_error() then describes the problem.
 *  - Results are bitwise deterministic from run to run.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef SEER_H_
#define SEER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum seer_status {
  SEER_OK = 0,
  SEER_ERR_INVALID_ARG = 1, /* null pointer where one is required, bad enum,
                               non-finite threshold, k < 1 */
  SEER_ERR_SHAPE = 2,       /* negative size, heads_q % heads_kv != 0,
                               block != 64, sizes whose tensors overflow */
  SEER_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, gate_dim not a multiple
                               of 16 in [16, 256], too many blocks per row */
  SEER_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the query */
  SEER_ERR_HIP = 5          /* the HIP runtime reported an error */
} seer_status;

/* Problem sizes. block must be 64 (the gate's pooling window, which is also
 * the attention tile: [E] section 3.4, "Block-sparse FlashAttention kernel").
 * Zero sizes are valid and make a call a no-op. */
typedef struct seer_shape {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t seq_len;
  int32_t head_dim;
  int32_t block;
} seer_shape;

typedef enum seer_mask_mode {
  SEER_MASK_THRESHOLD = 0, /* b_ij = score_ij > T           ([E] 3.4 Method 2) */
  SEER_MASK_TOPK = 1       /* k largest scores of row i      ([E] 3.4 Method 1) */
} seer_mask_mode;

typedef enum seer_dtype { SEER_F32 = 0, SEER_BF16 = 1 } seer_dtype;

/* ------------------------------------------------------------------------
 * AttnGate ([E] section 3.4, "AttnGate: The Learned Sparsity Predictor" and
 * its score equation; "Pooling Method Selection"; "Inference Procedure",
 * Methods 1 and 2; [R] response 3.3 on mask generation).
 *
 *   Qp[b,h,i]  = mean of Q[b,h,t] over the tokens t of block i        ([B,Hq,nb,D])
 *   Kp[b,g,i]  = [max | min | mean] of K[b,g,t] over block i          ([B,Hkv,nb,3D])
 *   Q'[b,h,i]  = Qp[b,h,i] . w_q[h]                                    (D -> gate_dim)
 *   K'[b,h,j]  = Kp[b,g(h),j] . w_k[h]   (w_k per query head), or
 *               Kp[b,g(h),j] . w_k[g(h)] (wk_per_kv_head != 0)        (3D -> gate_dim)
 *   with rope_theta > 0 (block-level RoPE, [E] section 3.4 "Block-Level
 *   RoPE"; q and k are then the model's Q and K BEFORE its own rotary
 *   embedding): Q'_i and K'_j are rotated at their block positions i and j,
 *   dims d and d + gate_dim/2 forming a pair, by the angle
 *   pos * (rope_theta / 64)^(-2d / gate_dim)  (the model's RoPE base divided
 *   by the block size); rope_theta = 0 leaves them unrotated
 *   score[b,h,i,j] = softmax over j <= i of Q'_i . K'_j / sqrt(D); 0 for j > i
 *   mask[b,h,i,j]  = 1 if the block is selected, else 0 (also 0 for j > i)
 *     threshold: score > threshold (strict)
 *     top-k    : the k largest causal scores of row i, ties to the lower j;
 *                a row with i+1 <= k keeps all its causal blocks
 *   Everything is computed in fp32; the mask is decided on the fp32 scores.
 *
 * q            device bf16 [B,Hq,S,D]
 * k            device bf16 [B,Hkv,S,D]
 * w_q          device fp32 [Hq,D,gate_dim]
 * w_k          device fp32 [Hq,3D,gate_dim] or [Hkv,3D,gate_dim]
 * rope_theta   0, or the base of the model's RoPE (> 0, finite), e.g. 500000
 * threshold    used in SEER_MASK_THRESHOLD mode; must be finite
 * topk_k       uniform k for SEER_MASK_TOPK (>= 1) when topk_per_head is NULL
 * topk_per_head HOST array of Hq values of k (>= 1), or NULL; read during the call
 * scores       device fp32 [B,Hq,nb,nb] output, or NULL if not wanted
 * block_mask   device uint8 [B,Hq,nb,nb] output (required)
 * workspace    device scratch of at least seer_gate_workspace_size() bytes
 * ---------------------------------------------------------------------- */
size_t seer_gate_workspace_size(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head,
                                int32_t want_scores);
seer_status seer_gate_fwd(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head,
                          float rope_theta, const void* q, const void* k, const float* w_q, const float* w_k,
                          seer_mask_mode mode, float threshold, int32_t topk_k,
                          const int32_t* topk_per_head, float* scores, uint8_t* block_mask,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * One self-distillation step of the gate ([E] section 3.4, "Training
 * Procedure": loss = D_KL(gt || score), gt the 2D-maxpooled attention map of
 * seer_attn_maxpool_gt and score the gate's output, both read as
 * distributions over the key blocks of a query block).
 *
 *   score      = the gate score of seer_gate_fwd (same q, k, weights, rope_theta)
 *   p[b,h,i,:] = gt[b,h,i,j] / sum_{j<=i} gt[b,h,i,j] over the causal entries
 *   loss       = (1 / (B Hq nb)) * sum_{b,h,i} sum_{j<=i, p>0} p log(p / score)
 *   grad_wq    = d loss / d w_q,  grad_wk = d loss / d w_k   (overwritten)
 *   A row of gt whose causal entries sum to 0 adds 0 to the loss and to the
 *   gradients. Everything is computed in fp32; the loss is summed in fp64.
 *
 * gt           device fp32 [B,Hq,nb,nb] (entries above the diagonal ignored)
 * loss         device fp32 [1] output
 * grad_wq      device fp32 [Hq,D,gate_dim] output
 * grad_wk      device fp32, shaped like w_k, output
 * workspace    device scratch of at least seer_gate_distill_workspace_size()
 *              bytes, 256-byte aligned
 * Other arguments as for seer_gate_fwd.
 * ---------------------------------------------------------------------- */
size_t seer_gate_distill_workspace_size(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head);
seer_status seer_gate_distill_bwd(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head,
                                  float rope_theta, const void* q, const void* k, const float* w_q,
                                  const float* w_k, const float* gt, float* loss, float* grad_wq,
                                  float* grad_wk, void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/* ------------------------------------------------------------------------
 * Causal GQA block-sparse attention forward ([E] section 3.4, "Block-sparse
 * FlashAttention kernel": a tile whose mask entry is 0 is skipped whole -- no
 * Q.K^T, no softmax, no P.V and no K/V loads -- and a tile whose entry is 1 is
 * computed as in FlashAttention-2; [R] response 3.3: blocks marked True are
 * activated in the kernel).
 *
 *   O[b,h,t]  = sum_u softmax_u(Q[b,h,t] . K[b,g,u] / sqrt(D)) V[b,g,u]
 *               over keys u <= t whose block is active in mask[b,h,t/64,u/64]
 *   lse[b,h,t] = natural-log sum of exp of those logits
 *   A query with no active key gets O = 0 and lse = -inf.
 *
 * block_mask   device uint8 [B,Hq,nb,nb]; any non-zero byte means "compute";
 *              entries above the diagonal are ignored. NULL = dense causal
 *              attention over every block (the speedup denominator).
 * out          device [B,Hq,S,D] in out_dtype (fp32 or bf16)
 * lse          device fp32 [B,Hq,S] output, or NULL
 * workspace    device scratch of at least seer_attn_workspace_size() bytes,
 *              16-byte aligned, used only when block_mask is non-NULL. Rows
 *              of at least 960 blocks with at least 64 (batch, KV head,
 *              128-block chunk) pairs are processed in key chunks of 128
 *              blocks, each owned by one XCD: the chunks before a row's
 *              diagonal chunk leave partial outputs there, which the diagonal
 *              chunk's pass merges; 64 * (2 * head_dim + 4) bytes per row and
 *              chunk it reaches (bf16 output, fp32 log-sum-exp) plus 256 bytes
 *              of item counters that every call resets. Other rows of more
 *              than 1024 blocks (seq_len > 65536) use key chunks of 512
 *              blocks whose partials a second kernel merges:
 *              64 * (head_dim + 1) * 4 bytes per row and chunk. Rows of at
 *              most 256 blocks at head_dim 128 (512 at head_dim 64) with
 *              batch * heads_q a multiple of 8 take 256 bytes: a pre-pass
 *              counts the mask's active tiles per XCD of the XCD-major row
 *              order (each XCD takes an eighth of the heads), which is used
 *              when those counts are balanced. Other rows of 257 to 1024
 *              blocks at head_dim 128 with batch * heads_q * blocks >= 8192
 *              also take 256 bytes: the per-XCD row queues of a persistent
 *              launch, which every call resets. Otherwise the size is 0 and
 *              workspace may be NULL. The active blocks of each row are
 *              compacted on chip.
 * ---------------------------------------------------------------------- */
size_t seer_attn_workspace_size(const seer_shape* shape);
seer_status seer_block_sparse_attn_fwd(const seer_shape* shape, const void* q, const void* k,
                                       const void* v, const uint8_t* block_mask, void* out,
                                       seer_dtype out_dtype, float* lse, void* workspace,
                                       size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Dense causal attention that also emits the 2D-maxpooled attention map, the
 * gate's distillation target ([E] section 3.4, "Training Procedure": gt
 * equation and the customized training kernel that stores the per-tile row
 * maxima r_ij, rescales them with the final row statistics and takes a
 * column max).
 *
 *   gt[b,h,i,j] = max over t in block i, u in block j, u <= t of
 *                 softmax_u(Q[b,h,t] . K[b,g,u] / sqrt(D));  0 for j > i
 *   (raw max-pooled probabilities, not renormalized)
 *
 * out, lse     as for seer_block_sparse_attn_fwd with block_mask = NULL
 * gt           device fp32 [B,Hq,nb,nb] output (required)
 * workspace    device scratch of at least seer_gt_workspace_size() bytes
 *              (the stored per-row, per-key-block maxima)
 * ---------------------------------------------------------------------- */
size_t seer_gt_workspace_size(const seer_shape* shape);
seer_status seer_attn_maxpool_gt(const seer_shape* shape, const void* q, const void* k,
                                 const void* v, void* out, seer_dtype out_dtype, float* lse,
                                 float* gt, void* workspace, size_t workspace_bytes,
                                 void* hip_stream);

/* ------------------------------------------------------------------------
 * Decode stage ([R], the responses on decoding: for decode the gate drops the
 * query branch's pooling and linear map, each new token's query meets a small
 * compressed K cache -- keys pooled after the model's RoPE -- and only the
 * selected blocks' K and V are read; the gate is distilled against the
 * attention map max-pooled along the sequence).
 *
 * shape->seq_len is the number of cached tokens S (the newest token's key and
 * value included); nb = ceil(S / 64). The decode query q is [B,Hq,D] bf16,
 * the query of the newest token (after the model's RoPE); it sees every
 * cached key. k_cache, v_cache are [B,Hkv,S,D] bf16.
 *
 * seer_decode_compress_k: the compressed cache
 *   kcomp[b,w,j,:] = [max | min | mean]_{t in block j} K[b,g(w),t,:] . w_k[w]
 *   for blocks block_begin <= j < nb (the others are left as they are), with
 *   w_k fp32 [Hwk,3D,D], Hwk = Hq (g(w) = w / (Hq/Hkv)) or, with
 *   wk_per_kv_head, Hkv (g(w) = w). kcomp is device fp32
 *   [B,Hwk,kcomp_blocks,D] with kcomp_blocks >= nb (room to grow): after
 *   appending tokens, recompute from the first changed block.
 * seer_decode_gate_fwd: score[b,h,j] = softmax over all j < nb of
 *   q[b,h] . kcomp[b,w(h),j] / sqrt(D) (w(h) = h, or h / (Hq/Hkv) with
 *   wk_per_kv_head); block_mask [B,Hq,nb] uint8 = score > threshold, or the
 *   top-k per (b,h) (ties to the lower j, all blocks if nb <= k); scores
 *   [B,Hq,nb] fp32 (required: it holds the logits, then the scores).
 *   q and kcomp 16-byte aligned. nb <= 16384. No workspace.
 * seer_decode_attn_fwd: O[b,h] = sum_u softmax_u(q[b,h] . K[b,g,u] / sqrt(D))
 *   V[b,g,u] over the keys of the blocks active in block_mask[b,h,:] (NULL:
 *   every block); out [B,Hq,D] in out_dtype, lse [B,Hq] (natural log) or
 *   NULL; a head with no active block gets O = 0, LSE = -inf. With
 *   block_mask NULL, gt (fp32 [B,Hq,nb], or NULL) receives the 1D max-pooled
 *   map gt[b,h,j] = max_{u in block j} softmax_u(...); gt must be NULL when a
 *   mask is given. A block no query head of a KV group selects is not read.
 *   Hq/Hkv <= 8. workspace: seer_decode_attn_workspace_size() bytes,
 *   16-byte aligned (per-split partial results).
 * ---------------------------------------------------------------------- */
seer_status seer_decode_compress_k(const seer_shape* shape, int32_t wk_per_kv_head, const void* k_cache,
                                   const float* w_k, int32_t block_begin, float* kcomp, int32_t kcomp_blocks,
                                   void* hip_stream);
seer_status seer_decode_gate_fwd(const seer_shape* shape, int32_t wk_per_kv_head, const void* q,
                                 const float* kcomp, int32_t kcomp_blocks, seer_mask_mode mode,
                                 float threshold, int32_t topk_k, const int32_t* topk_per_head,
                                 float* scores, uint8_t* block_mask, void* hip_stream);
size_t seer_decode_attn_workspace_size(const seer_shape* shape);
seer_status seer_decode_attn_fwd(const seer_shape* shape, const void* q, const void* k_cache,
                                 const void* v_cache, const uint8_t* block_mask, void* out,
                                 seer_dtype out_dtype, float* lse, float* gt, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Allocation-free decode attention, for callers that cannot allocate device
 * memory between calls: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Computes exactly what seer_decode_attn_fwd computes (same kernels, same
 * bits), with the same arguments minus the workspace. Its scratch (per-split
 * partial results and the per-KV-group block lists) is a fixed array of
 * SEER_NOALLOC_SCRATCH_BYTES in each device's copy of the library, held until
 * the process ends; the call allocates nothing (no hipMalloc, no library
 * routine that allocates). Shapes whose seer_decode_attn_workspace_size()
 * exceeds SEER_NOALLOC_SCRATCH_BYTES are rejected with SEER_ERR_UNSUPPORTED
 * before anything is enqueued (16 MiB covers, e.g., batch 64 of 32/8 heads
 * at 128k cached tokens). Every call on one device shares that device's
 * scratch and overwrites it: calls that can overlap on one device (other
 * streams, other threads) race and must be serialized by the caller. No
 * part of the scratch has to start at zero.
 * ---------------------------------------------------------------------- */
#define SEER_NOALLOC_SCRATCH_BYTES (16u << 20)
seer_status seer_decode_attn_fwd_noalloc(const seer_shape* shape, const void* q, const void* k_cache,
                                         const void* v_cache, const uint8_t* block_mask, void* out,
                                         seer_dtype out_dtype, float* lse, float* gt, void* hip_stream);

/* ------------------------------------------------------------------------
 * Varlen (packed) prefill batches ([R], on batching: variable-length inputs
 * are packed along the sequence dimension, hiding the batch in the sequence
 * length).
 *
 * num_seqs sequences are packed without padding: sequence i is tokens
 * cu_seqlens[i] .. cu_seqlens[i+1]-1 of T = cu_seqlens[num_seqs] tokens.
 * Tensors are head-major over the packed tokens: q [Hq,T,D], k and v
 * [Hkv,T,D] bf16; out [Hq,T,D]; lse [Hq,T]. Each sequence keeps its own
 * 64-token blocks (the gate never pools across sequences, attention never
 * crosses them), so its block maps (scores, mask, gt) are [Hq,nb_i,nb_i],
 * nb_i = ceil(len_i / 64), stored one after another: sequence i's map starts
 * at element sum_{i'<i} Hq * nb_i'^2 (seer_varlen_map_elements() gives the
 * total). Every call computes exactly what the batch-1 call computes on each
 * sequence alone, bit for bit. Attention and the ground-truth map run the
 * sequences together: up to 64 sequences per launch, longest first, each row
 * of each sequence one workgroup of a single grid (in block-sparse mode,
 * sequences of more than 1024 blocks run on their own launches, key-chunked,
 * and share the workspace). The gate runs runs of up to 64 consecutive
 * sequences of at most 4096 blocks each in one launch per stage; a longer
 * sequence ends a run and runs on its own launches. Its workspace
 * (seer_gate_varlen_workspace_size()) holds the largest run's intermediates
 * side by side. seer_gt_varlen_workspace_size() covers the scratch of every
 * sequence of the largest shared launch; the attention workspace is the
 * largest any sequence needs. All sequences are validated, and the
 * workspace checked, before anything is enqueued. Empty sequences are
 * allowed.
 * ---------------------------------------------------------------------- */
typedef struct seer_varlen {
  int32_t num_seqs;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int32_t block;                /* must be 64 */
  const int32_t* cu_seqlens;    /* HOST array of num_seqs + 1 non-decreasing offsets, cu_seqlens[0] = 0 */
} seer_varlen;

size_t seer_varlen_map_elements(const seer_varlen* vl);
size_t seer_gate_varlen_workspace_size(const seer_varlen* vl, int32_t gate_dim, int32_t wk_per_kv_head,
                                       int32_t want_scores);
seer_status seer_gate_varlen_fwd(const seer_varlen* vl, int32_t gate_dim, int32_t wk_per_kv_head,
                                 float rope_theta, const void* q, const void* k, const float* w_q,
                                 const float* w_k, seer_mask_mode mode, float threshold, int32_t topk_k,
                                 const int32_t* topk_per_head, float* scores, uint8_t* block_mask,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);
size_t seer_attn_varlen_workspace_size(const seer_varlen* vl);
seer_status seer_block_sparse_attn_varlen_fwd(const seer_varlen* vl, const void* q, const void* k,
                                              const void* v, const uint8_t* block_mask, void* out,
                                              seer_dtype out_dtype, float* lse, void* workspace,
                                              size_t workspace_bytes, void* hip_stream);
size_t seer_gt_varlen_workspace_size(const seer_varlen* vl);
seer_status seer_attn_maxpool_gt_varlen(const seer_varlen* vl, const void* q, const void* k, const void* v,
                                        void* out, seer_dtype out_dtype, float* lse, float* gt,
                                        void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * seer_status_string: static name of a status code.
 * seer_last_error: message of the last failing call on this thread ("" if
 *   none); valid until the next call on this thread.
 * seer_version: library version string.
 * ---------------------------------------------------------------------- */
const char* seer_status_string(seer_status status);
const char* seer_last_error(void);
const char* seer_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEER_H_ */
