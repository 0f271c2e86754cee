/*
 * chunk_kda: the KDA attention recurrence of the K3 notes, as a C ABI over
 * device pointers (gfx950 HIP library, same shared object as mla_absorb.h).
 *
 * Definition (page "符号表": section KDA 变量 for the variables and their
 * shapes, section Einsum 速查 for the contractions, and the summary list on
 * that page: the chunked evaluation equals the step-by-step recurrence).
 * Per batch b and value head hv, with query/key head h = hv / G (grouped
 * value attention: H_V = G H value heads share H query/key heads) and the
 * state S [K, V] starting at the initial state (zero when it is NULL), for
 * t = 0 .. T-1:
 *   S   = diag(exp(g_t)) S            decay per key channel (g is log-space)
 *   r_t = v_t - k_t^T S               delta-rule residual of the old state
 *   S   = S + (beta_t k_t) r_t^T      write
 *   o_t = q_t^T S                     read-out after the write
 * q already carries the attention scale (the pages' table says so); the gate
 * activation that produces g is not part of this call.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#include "mla_absorb.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Bytes of workspace kda_chunk_forward needs ((size_t)-1 for invalid sizes or
 * an unsupported dtype).  It grows with B * G * H * ceil(T / 64): about 81 KiB
 * per (batch, value head, 64 positions) at K = V = 128.
 */
size_t kda_chunk_workspace_size(int B, int T, int H, int G, int K, int V, mla_dtype dtype);

/*
 * chunk_kda forward over B sequences of T positions each.
 *   q, k           [B, T, H, K]    bf16, row-major
 *   v              [B, T, G*H, V]  bf16
 *   g              [B, T, G*H, K]  float32, log-space decay, each in [-5, 0]
 *                                  (the gate's lower bound on the pages; the
 *                                  chunked evaluation keeps every exponent in
 *                                  range down to about -5.9 per step)
 *   beta           [B, T, G*H]     float32 write strength
 *   initial_state  [B, G*H, K, V]  float32, or NULL for a zero state
 *   o              [B, T, G*H, V]  bf16 output (written)
 *   final_state    [B, G*H, K, V]  float32 (written), or NULL
 * Supported head widths: K = V in {16, 64, 128}; dtype MLA_DTYPE_BF16 only;
 * one batch's g must stay under 2e9 bytes (MLA_ERR_UNSUPPORTED otherwise).  Positions are processed in chunks of 64
 * (the last one may be partial).  The caller owns every buffer; workspace is
 * kda_chunk_workspace_size bytes, 16-byte aligned (MLA_ERR_WORKSPACE
 * otherwise).  All pointers are device pointers, 16-byte aligned
 * (MLA_ERR_INVALID_ARG for a null or misaligned required pointer or a
 * non-positive size).  Launches on `stream` (a hipStream_t, NULL for the
 * default stream); no allocation, no synchronisation.
 */
mla_status kda_chunk_forward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* initial_state, void* o, float* final_state, int B, int T, int H, int G,
                             int K, int V, mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
