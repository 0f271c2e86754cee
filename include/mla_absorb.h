/*
 * mla_absorb.h - C ABI of the MI355X (gfx950) library for the matrix-absorbed,
 * NoPE Gated MLA attention layer.
 *
 * The layer (page "Gated MLA（矩阵吸收版）" of the K3 notes: sections 低秩压缩,
 * 矩阵吸收的核心思路, 完整计算流（四步） steps 2-4 and the 代码对照 listing;
 * shapes from page "符号表", section MLA 变量) computes for every batch b,
 * head h and query position t:
 *
 *   q_abs[b,t,h,:] = q[b,t,h,:] . W_UK[h]                 (absorb W_UK, [r])
 *   score[b,h,t,s] = scale * q_abs[b,t,h,:] . c[b,s,:]     (latent score)
 *   attn           = softmax over s of score, keys s > t masked (causal)
 *   o_lat[b,h,t,:] = sum_s attn[b,h,t,s] * c[b,s,:]        (latent weighted sum, [r])
 *   o[b,h,t,v]     = o_lat[b,h,t,:] . W_UV[h,v,:]           (W_UV^T up-projection)
 *   out[b,t,h*d_v+v] = sigmoid(gate[b,t,h*d_v+v]) * o[b,h,t,v]
 *
 * The pages print no softmax scale, so it is an explicit argument.  The
 * output is the gated, head-major flattened tensor before the output
 * projection.  Decode evaluates the same definition for one new query per
 * sequence against a packed latent cache (the pages cache only c; the decode
 * path itself is not written on the pages).
 *
 * Conventions for every entry point:
 *  - All tensors are device pointers to row-major contiguous storage, all of
 *    the same element type (dtype), 16-byte aligned.  cu_seqlens is int32.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises; scratch memory comes from the caller's workspace, whose
 *    size the *_workspace_size functions return.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the null
 *    stream) and the call returns without waiting.  MLA_OK means enqueued.
 *  - Arguments are checked on the host before anything is launched:
 *    MLA_ERR_INVALID_ARG (null or misaligned pointer, non-positive size,
 *    non-finite scale), MLA_ERR_UNSUPPORTED ((d_q, d_v, r) outside the
 *    compiled set for bf16, or sizes beyond the int32 index range),
 *    MLA_ERR_WORKSPACE (workspace smaller than required).  A launch failure
 *    reported by the HIP runtime returns MLA_ERR_HIP.
 *  - Inputs are read only.  `out` must not alias any input or the workspace.
 *  - Calls may run concurrently on different streams with distinct
 *    workspaces.  The only global state is the scratch buffer of
 *    mla_absorb_decode_noalloc (one per GPU) and the cached device address
 *    of it, resolved once per device under a lock.
 *
 * Supported element types: MLA_DTYPE_BF16 (bf16 storage, fp32 accumulation,
 * MFMA kernels; (d_q, d_v, r) in {(16,16,32), (64,64,256), (128,128,512)}) and
 * MLA_DTYPE_F32 (fp32 throughout; any d_q, d_v <= 256 and r <= 1024).
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE = 3,
  MLA_ERR_HIP = 4
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status s);

/*
 * Bytes of workspace mla_absorb_prefill needs for these sizes (0 is a valid
 * answer).  Returns (size_t)-1 for invalid sizes.  The bf16 workspace holds
 * W_UK transposed per head and a work-item counter that the call itself
 * clears before use; calls that overlap on one workspace race.
 */
size_t mla_absorb_prefill_workspace_size(int B, int T, int H, int d_q, int r, mla_dtype dtype);

/*
 * Prefill: causal attention of every position of B sequences of length T.
 *   q     [B, T, H, d_q]   queries (output of the query low-rank path)
 *   c     [B, T, r]        KV latent, shared by all heads
 *   w_uk  [H, d_q, r]      key decompression W_UK (the first H*d_q rows of
 *                          kv_up.weight viewed as [H, d_q, r])
 *   w_uv  [H, d_v, r]      value decompression W_UV (the following H*d_v rows)
 *   gate  [B, T, H*d_v]    gate pre-activations (before the sigmoid)
 *   out   [B, T, H*d_v]    gated output, column h*d_v + v
 *   scale                  softmax scale applied to q_abs . c
 */
mla_status mla_absorb_prefill(const void* q, const void* c, const void* w_uk, const void* w_uv,
                              const void* gate, void* out, int B, int T, int H, int d_q, int d_v,
                              int r, float scale, mla_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Chunked prefill against a cached prefix: the T queries of each sequence are
 * its positions S-T .. S-1, and query t attends to latent rows 0 .. S-T+t
 * (the causal softmax of page "Gated MLA（矩阵吸收版）", section
 * 完整计算流（四步） step 2, for a chunk that follows S-T positions already in
 * the latent cache; the pages cache only c, section 低秩压缩).  Prefill is the
 * case S == T; a one-query chunk (T == 1) is a decode step.
 *   q     [B, T, H, d_q]   queries of the chunk
 *   c     [B, S, r]        latent of every position of each sequence,
 *                          prefix first, the chunk's own rows last
 *   gate, out [B, T, H*d_v]
 *   w_uk, w_uv, scale      as for prefill
 * Workspace: mla_absorb_prefill_workspace_size(B, T, H, d_q, r, dtype) bytes.
 * Errors as for prefill; S < T is MLA_ERR_INVALID_ARG.
 */
mla_status mla_absorb_extend(const void* q, const void* c, const void* w_uk, const void* w_uv,
                             const void* gate, void* out, int B, int T, int S, int H, int d_q, int d_v,
                             int r, float scale, mla_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace mla_absorb_decode needs.  num_splits <= 0 selects the
 * library default (the device's compute-unit count, which queries the
 * current device).  Returns (size_t)-1 for invalid sizes.
 */
size_t mla_absorb_decode_workspace_size(int B, int H, int d_q, int r, int num_splits,
                                        mla_dtype dtype);

/*
 * Workspace of mla_absorb_prefill (is_decode = 0, T_or_max_len = T) or of
 * mla_absorb_decode with the default split count (is_decode != 0;
 * T_or_max_len, the longest cache, bounds nothing there and only has to be
 * positive, because decode splits the packed cache rows evenly whatever the
 * lengths).  d_q is implied by r: the compiled bf16 set pairs r = 32, 256,
 * 512 with d_q = 16, 64, 128.  Returns 0 for MLA_DTYPE_F32 and (size_t)-1
 * for invalid sizes, an r outside the compiled set, or (decode) when no
 * device can be queried for its compute-unit count.  The calls with explicit
 * head widths and split counts are mla_absorb_prefill_workspace_size and
 * mla_absorb_decode_workspace_size.
 */
size_t mla_absorb_workspace_size(int is_decode, int B, int T_or_max_len, int H, int r, mla_dtype dtype);

/*
 * Decode: one new query per sequence against a packed latent cache.
 *   q          [B, H, d_q]      the query of each sequence, at position len_i - 1
 *   c_cache    [total_len, r]   latents of all sequences back to back; sequence
 *                               i owns rows cu_seqlens[i] .. cu_seqlens[i+1]-1,
 *                               the last of which is the new token's own latent
 *   cu_seqlens [B + 1] int32    device array, exclusive prefix sums of the
 *                               lengths: cu_seqlens[0] = 0,
 *                               cu_seqlens[B] = total_len, every length >= 1
 *                               (a precondition; it is not read on the host)
 *   w_uk, w_uv                  as for prefill
 *   gate       [B, H*d_v]       gate pre-activations
 *   out        [B, H*d_v]       gated output
 *   total_len                   rows of c_cache (host value); every cache
 *                               access is clamped below it
 *   num_splits                  workgroups sharing the cache rows evenly
 *                               (<= 0: library default); any value gives the
 *                               same result up to rounding order
 * The split is stream-K over the packed rows (each workgroup takes
 * total_len / num_splits consecutive rows, across sequence boundaries), so
 * the grid depends on total_len and not on the longest sequence: the call
 * takes total_len, where a per-sequence split would take the maximum length.
 */
mla_status mla_absorb_decode(const void* q, const void* c_cache, const int32_t* cu_seqlens,
                             const void* w_uk, const void* w_uv, const void* gate, void* out,
                             int B, int H, int d_q, int d_v, int r, int64_t total_len, float scale,
                             int num_splits, mla_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the per-GPU static scratch buffer of mla_absorb_decode_noalloc. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * mla_absorb_decode (same arguments, kernels and result), but its scratch
 * (q_abs and the split partials) lives in a static device buffer of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * from the first call on that device until the process ends.  The call
 * allocates and frees nothing.  Sizes whose scratch exceeds the buffer
 * (mla_absorb_decode_workspace_size(B, H, d_q, r, num_splits, dtype) >
 * MLA_NOALLOC_SCRATCH_BYTES; e.g. B = 128 sequences at H = 96, r = 512 and
 * the default 256 splits need 48.3 MiB) return MLA_ERR_WORKSPACE before
 * anything is launched.  Every call on one GPU shares that GPU's buffer:
 * calls that overlap on one GPU (different streams, or different host
 * threads) race and give undefined results; serialise them.  Nothing in the
 * buffer needs to start at zero: each call writes every scratch byte it
 * reads.  Errors otherwise as for mla_absorb_decode; MLA_ERR_HIP also if the
 * buffer's address cannot be resolved on the current device.
 */
mla_status mla_absorb_decode_noalloc(const void* q, const void* c_cache, const int32_t* cu_seqlens,
                                     const void* w_uk, const void* w_uv, const void* gate, void* out,
                                     int B, int H, int d_q, int d_v, int r, int64_t total_len, float scale,
                                     int num_splits, mla_dtype dtype, void* stream);

/*
 * Paged latent cache (the pages cache only c, page "Gated MLA（矩阵吸收版）",
 * section 低秩压缩; how the cache is stored is not on the pages).  A pool
 *   c_pages [num_pages, page_size, r]
 * holds the rows of every sequence in fixed-size pages; row u of sequence i
 * is page block_table[i * max_pages + u / page_size], slot u % page_size.
 * block_table is an int32 device array [B, max_pages].  page_size is a power
 * of two, at least 32 (the key tile, so no tile crosses a page).  Page
 * indices are device data and are not read on the host: an entry outside
 * [0, num_pages) that a call needs reads as zero rows (append: the row is
 * skipped); nothing outside the pool is ever accessed.
 *
 * Chunked prefill over a paged cache: as mla_absorb_extend, with the S rows
 * of each sequence in pages (S <= max_pages * page_size).  bf16 only (f32 is
 * MLA_ERR_UNSUPPORTED).  Workspace: mla_absorb_prefill_workspace_size(B, T,
 * H, d_q, r, dtype) bytes.
 */
mla_status mla_absorb_extend_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                   const void* w_uk, const void* w_uv, const void* gate, void* out, int B, int T,
                                   int S, int H, int d_q, int d_v, int r, int64_t num_pages, int page_size,
                                   int max_pages, float scale, mla_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_absorb_extend_varlen_paged needs ((size_t)-1: invalid). */
size_t mla_absorb_extend_varlen_workspace_size(int B, int Nq, int H, int d_q, int r, mla_dtype dtype);

/*
 * Varlen chunked prefill over a paged cache: one call for a batch that mixes
 * full prefills, chunks after a cached prefix and single decode steps.
 * Sequence b owns the packed query rows cu_q[b] .. cu_q[b+1]-1 (T_b rows,
 * possibly none) and seq_lens[b] = S_b cache rows, its chunk being positions
 * S_b - T_b .. S_b - 1 (so query t attends to rows 0 .. S_b - T_b + t):
 *   q     [Nq, H, d_q]     queries of all chunks, sequence by sequence
 *   cu_q  [B + 1] int32    device array, cu_q[0] = 0, cu_q[B] = Nq, non-decreasing
 *   seq_lens [B] int32     device array, T_b <= S_b <= max_pages * page_size
 *   gate, out [Nq, H*d_v]
 *   c_pages, block_table   as for the paged calls (the chunk's own rows are in
 *                          the cache already, e.g. through mla_cache_append_paged)
 * cu_q and seq_lens are read on the device only: ranges are clamped into
 * [0, Nq) and [0, max_pages * page_size] before use, so a violated
 * precondition yields unspecified values for the affected rows, never an
 * access outside the buffers.  bf16 only.  Workspace:
 * mla_absorb_extend_varlen_workspace_size bytes.
 */
mla_status mla_absorb_extend_varlen_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                          const int32_t* cu_q, const int32_t* seq_lens, const void* w_uk,
                                          const void* w_uv, const void* gate, void* out, int B, int Nq, int H, int d_q,
                                          int d_v, int r, int64_t num_pages, int page_size, int max_pages, float scale,
                                          mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_absorb_decode_paged needs ((size_t)-1: invalid). */
size_t mla_absorb_decode_paged_workspace_size(int B, int H, int d_q, int r, int num_splits, mla_dtype dtype);

/*
 * Decode over a paged cache: as mla_absorb_decode, with sequence i's
 * seq_lens[i] rows (int32 device array [B], the new token's own row
 * included) in pages.  Lengths are clamped to [1, max_pages * page_size] on
 * the device.  bf16 only.  The stream-K split works in 32-row tiles of each
 * sequence; num_splits as for mla_absorb_decode.
 */
mla_status mla_absorb_decode_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                   const int32_t* seq_lens, const void* w_uk, const void* w_uv, const void* gate,
                                   void* out, int B, int H, int d_q, int d_v, int r, int64_t num_pages,
                                   int page_size, int max_pages, float scale, int num_splits, mla_dtype dtype,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cache append: writes row c_new[i] ([B, r], dtype) as row positions[i]
 * (int32 device array [B]) of sequence i of the paged cache, in place; the
 * row a decode step adds before it attends.  Any page size >= 1 works here;
 * r * sizeof(dtype) must be a multiple of 16 bytes.  A position outside
 * [0, max_pages * page_size) skips the row.  No workspace.
 */
mla_status mla_cache_append_paged(const void* c_new, void* c_pages, const int32_t* block_table,
                                  const int32_t* positions, int B, int r, int64_t num_pages, int page_size,
                                  int max_pages, mla_dtype dtype, void* stream);

/*
 * Training forward: mla_absorb_prefill that also writes, for the backward,
 *   lse [B, H, T] float32   log sum_{s<=t} exp(scale * q_abs[b,t,h,:] . c[b,s,:])
 * (natural log; the normaliser of the causal softmax).  bf16 only.  Other
 * arguments, workspace and errors as for mla_absorb_prefill.
 */
mla_status mla_absorb_prefill_train(const void* q, const void* c, const void* w_uk, const void* w_uv,
                                    const void* gate, void* out, float* lse, int B, int T, int H, int d_q, int d_v,
                                    int r, float scale, mla_dtype dtype, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Bytes of workspace mla_absorb_prefill_backward needs ((size_t)-1: invalid). */
size_t mla_absorb_prefill_backward_workspace_size(int B, int T, int H, int d_q, int d_v, int r, mla_dtype dtype);

/*
 * Backward of the prefill core.  The pages train the layer with a
 * cross-entropy loss; these are the gradients of the forward above (chain
 * rule through absorb, latent score, causal softmax, latent sum, W_UV and the
 * sigmoid gate) given dout = dLoss/dout.  c is both the key and the value of
 * the latent attention, so dc carries both paths, summed over heads.
 *   inputs:  q, c, w_uk, w_uv, gate as for the forward; out [B, T, H*d_v] and
 *            lse [B, H, T] from mla_absorb_prefill_train; dout [B, T, H*d_v]
 *   outputs: dq [B, T, H, d_q], dc [B, T, r], dgate [B, T, H*d_v] (bf16) and
 *            dw_uk [H, d_q, r], dw_uv [H, d_v, r] (float32, overwritten)
 * bf16 only, (d_q, d_v, r) in the compiled set; the head-major intermediates
 * must stay below 2 GB each (H * B * T * r * 2 bytes), else
 * MLA_ERR_UNSUPPORTED.  Workspace: mla_absorb_prefill_backward_workspace_size
 * bytes (about 4 * H * B * T * r * 2 bytes).  Other conventions as above.
 */
mla_status mla_absorb_prefill_backward(const void* q, const void* c, const void* w_uk, const void* w_uv,
                                       const void* gate, const void* out, const float* lse, const void* dout,
                                       void* dq, void* dc, float* dw_uk, float* dw_uv, void* dgate, int B, int T,
                                       int H, int d_q, int d_v, int r, float scale, mla_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace mla_gated_forward needs (bf16 only; (size_t)-1 for
 * invalid sizes or dtypes).
 */
size_t mla_gated_forward_workspace_size(int B, int T, int q_rank, int H, int d_q, int d_v, int r,
                                        mla_dtype dtype);

/*
 * Full Gated MLA forward around the absorbed core (page "Gated MLA（矩阵吸收版）":
 * section 低秩压缩 for the latent, section 完整计算流（四步） steps 1-4):
 *   c    = RMSNorm(x W_kv_down^T) * kv_norm            [B, T, r]
 *   q    = (RMSNorm(x W_q_down^T) * q_norm) W_q_up^T    [B, T, H*d_q]
 *   gate = x W_gate^T                                   [B, T, H*d_v]
 *   o    = the absorbed core (mla_absorb_prefill) of q, c, W_UK, W_UV, gate
 *   y    = o W_o^T                                      [B, T, D]
 * with RMSNorm(v) = v / sqrt(mean(v^2) + eps) over the last axis.  Weights
 * are laid out as linear layers (out_features x in_features):
 *   w_kv_down [r, D], kv_norm [r], w_q_down [q_rank, D], q_norm [q_rank],
 *   w_q_up [H*d_q, q_rank], w_uk [H, d_q, r], w_uv [H, d_v, r],
 *   w_gate [H*d_v, D], w_o [D, H*d_v]; x and y are [B, T, D].
 * bf16 only (MLA_ERR_UNSUPPORTED otherwise).  The projections run as 64-wide
 * k tiles: D, q_rank and H*d_v must be multiples of 64, and r, q_rank <= 2048.
 * Workspace: mla_gated_forward_workspace_size bytes.  Other conventions and
 * errors as for mla_absorb_prefill.
 */
mla_status mla_gated_forward(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                             const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                             const void* w_gate, const void* w_o, void* y, int B, int T, int D, int q_rank,
                             int H, int d_q, int d_v, int r, float eps, float scale, mla_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the saved state mla_gated_forward_train keeps for
 * mla_gated_backward (bf16 only; (size_t)-1 for invalid sizes or dtypes).
 */
size_t mla_gated_train_state_size(int B, int T, int q_rank, int H, int d_q, int d_v, int r, mla_dtype dtype);

/*
 * Training form of mla_gated_forward: the same y (same arithmetic, same
 * conventions and errors), and the caller-owned buffer `state`
 * (mla_gated_train_state_size bytes, 16-byte aligned) receives what the
 * backward reads: the inputs of the two RMSNorms and their 1/rms, their
 * outputs, q, the gate pre-activations, the gated core output and the
 * core's log-sum-exp (as mla_absorb_prefill_train).  The layout of `state`
 * is private to this library; it stays valid until the caller overwrites
 * it.  MLA_ERR_WORKSPACE if state is null, misaligned or too small.
 */
mla_status mla_gated_forward_train(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                                   const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                                   const void* w_gate, const void* w_o, void* y, int B, int T, int D, int q_rank,
                                   int H, int d_q, int d_v, int r, float eps, float scale, mla_dtype dtype,
                                   void* state, size_t state_bytes, void* stream);

/*
 * Bytes of workspace mla_gated_backward needs (bf16 only; (size_t)-1 for
 * invalid sizes or dtypes).
 */
size_t mla_gated_backward_workspace_size(int B, int T, int D, int q_rank, int H, int d_q, int d_v, int r,
                                         mla_dtype dtype);

/*
 * Backward of the full Gated MLA layer (page "Gated MLA（矩阵吸收版）":
 * section 低秩压缩 and section 完整计算流（四步） steps 1-4, differentiated by
 * the chain rule) given dy = dLoss/dy [B, T, D] and the `state` that
 * mla_gated_forward_train left for the same x and weights:
 *   output projection  dO = dy W_o,           dW_o = dy^T o
 *   core               dq, dc, dgate, dW_UK, dW_UV as mla_absorb_prefill_backward
 *   query path         dql = dq W_q_up,       dW_q_up = dq^T ql
 *   the two RMSNorms   u = g v rstd:  dv = (du g - n mean(du g n)) rstd with
 *                      n = v rstd, and dg = sum over tokens of du n
 *   products of x      dx = dgate W_gate + dql_pre W_q_down + dc_pre W_kv_down,
 *                      dW_gate = dgate^T x, dW_q_down = dql_pre^T x,
 *                      dW_kv_down = dc_pre^T x.
 * Weights and x as for mla_gated_forward; dy and dx bf16 [B, T, D]; every
 * parameter gradient is float32 in the shape of its parameter (dkv_norm [r],
 * dq_norm [q_rank]), written, not accumulated.  bf16 only; shape limits of
 * mla_gated_forward and of mla_absorb_prefill_backward.  MLA_ERR_INVALID_ARG
 * also for a null, misaligned or too small state; workspace:
 * mla_gated_backward_workspace_size bytes, 16-byte aligned.
 */
mla_status mla_gated_backward(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                              const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                              const void* w_gate, const void* w_o, const void* dy, const void* state,
                              size_t state_bytes, void* dx, float* dw_kv_down, float* dkv_norm, float* dw_q_down,
                              float* dq_norm, float* dw_q_up, float* dw_uk, float* dw_uv, float* dw_gate,
                              float* dw_o, int B, int T, int D, int q_rank, int H, int d_q, int d_v, int r,
                              float scale, mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
