/*
 * spec_verify.h - C ABI of the speculative-decoding verification sampler for MI355X (gfx950).
 *
 * The operation (defined on the pages "Speculative Speculative Decoding - асинхронизируй это",
 * SD recap: accept / reject / residual rule; "Accélérer Sonar par la Spéculation", sections
 * "Décodage spéculatif" and "Cible-Brouillon": n drafts give up to n + 1 tokens, the target's
 * logits after the accepted prefix are sampled for one more; "NVIDIA: öt irányelv ...",
 * section "Mit csinál a spekulatív dekódolás?": in-order acceptance up to the first mismatch,
 * AL in [1, 1 + D]):
 *
 *   For each sequence b with draft length L = L_b and temperature T = T_b:
 *     T > 0:  p_i = softmax(target[b][i] / T), q_i = softmax(draft[b][i] / T).
 *             For i = 0 .. L-1: accept draft token x_i iff u[b][i] < min(1, p_i(x_i)/q_i(x_i));
 *             stop at the first rejection j and draw the token at j from
 *             norm(max(0, p_j - q_j)); if all L are accepted, draw a bonus token from p_L.
 *             The draw is an inverse CDF in ascending token id with the uniform u[b][D]:
 *             the smallest k with sum_{v<=k} w_v > u[b][D] * sum_v w_v.
 *     T == 0: greedy: accept x_i iff x_i is the target argmax at i (lowest index on ties);
 *             emit the target argmax at the first mismatch, or at position L if all match.
 *   AL = (number of accepted drafts) + 1, in [1, L + 1].
 *
 * Memory: every pointer argument except `workspace`-less host scalars is DEVICE memory owned
 * by the caller, row-major and contiguous. Nothing is retained after the call's stream work
 * completes. The call only enqueues work on `stream` (NULL = the default stream) and never
 * synchronizes; read the outputs after synchronizing that stream.
 *
 * Layouts (e = 2 bytes for bf16, 4 for fp32; target and draft share one dtype):
 *   target_logits  [B][D+1][V]  target logits at the D draft positions and the tail position.
 *   draft_logits   [B][D][V]    draft logits at the D draft positions.
 *   draft_tokens   [B][D]       int32; entries at positions >= L_b are ignored.
 *   draft_lens     [B]          int32 L_b in [0, D]; NULL means every L_b = D. Rows at target
 *                               positions > L_b and draft positions >= L_b are never read.
 *   uniforms       [B][D+1]     fp32 in [0, 1): columns 0..D-1 are the accept tests of
 *                               positions 0..D-1, column D is the final-draw uniform.
 *   temperature    [B]          fp32; 0 = greedy, > 0 sampled.
 *   out_accept_len [B]          int32 AL; 0 marks a row whose inputs are invalid.
 *   out_tokens     [B][D+1]     int32; the first AL entries are the emitted tokens
 *                               (accepted drafts, then the final token), the rest -1.
 *
 * Errors:
 *   - Problems visible on the host return a negative sv_status and enqueue nothing:
 *     a NULL required pointer, B <= 0, D < 0, V <= 0, D > SV_MAX_D, or sizes whose element
 *     counts overflow 64 bits.
 *   - Per-row data errors found on the device mark only that row (AL = 0, tokens -1):
 *     L_b outside [0, D], T_b negative, NaN or infinite, a draft token outside [0, V) at a
 *     position < L_b.
 *   - A failed launch or allocation returns SV_EHIP / SV_ENOMEM.
 *   - Logits may be -inf (a masked token: probability 0); every row that is read must hold at
 *     least one finite logit. NaN or +inf logits give unspecified tokens (never an
 *     out-of-bounds access).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_EINVAL = -1,   /* bad argument (NULL pointer, size out of range) */
  SV_EDTYPE = -2,   /* unknown dtype code */
  SV_EHIP = -3,     /* a HIP runtime call or kernel launch failed */
  SV_ENODEV = -4,   /* no usable gfx950 device */
  SV_ENOMEM = -5,   /* workspace allocation failed or caller workspace too small */
  SV_ESCRATCH = -6, /* spec_verify_noalloc: the problem needs more than its fixed scratch */
} sv_status;

#define SV_MAX_D 31   /* largest draft length D accepted (positions 0..D fit one 32-bit mask) */

/* bf16 logits (bit patterns of bfloat16, 2 bytes each). Returns SV_OK or a negative sv_status.
 * Uses a library-owned workspace, one per (current device, stream) that calls the plain entry
 * points, allocated on first use and grown when a larger problem arrives. Growth is
 * stream-ordered (hipFreeAsync of the old buffer and hipMallocAsync of the new one on `stream`),
 * so the host never waits; on a stream under graph capture a call that would need to grow the
 * workspace returns SV_ENOMEM and enqueues nothing (make a first call before the capture, or use
 * spec_verify_ws). Each buffer is held until spec_verify_release(stream) or the end of the
 * process. Calls on one device are serialized by a mutex while they enqueue. */
int spec_verify_bf16(const void* target_logits, const void* draft_logits,
                     const int32_t* draft_tokens, const int32_t* draft_lens,
                     const float* uniforms, int B, int D, int V,
                     const float* temperature, int32_t* out_accept_len,
                     int32_t* out_tokens, hipStream_t stream);

/* Same operation on fp32 logits. */
int spec_verify_f32(const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* draft_lens,
                    const float* uniforms, int B, int D, int V,
                    const float* temperature, int32_t* out_accept_len,
                    int32_t* out_tokens, hipStream_t stream);

/* Bytes of device workspace one call of shape (B, D, V) needs (0 on bad sizes). */
size_t spec_verify_workspace_bytes(int B, int D, int V);

/* Same operation with caller-provided device workspace of at least
 * spec_verify_workspace_bytes(B, D, V) bytes, 256-byte aligned. dtype: 0 = fp32, 1 = bf16.
 * Nothing is allocated. The workspace needs no initialisation (each call writes every part
 * it reads) and must not be used by another call until this call's stream work has
 * completed. */
int spec_verify_ws(int dtype, const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const int32_t* draft_lens,
                   const float* uniforms, int B, int D, int V,
                   const float* temperature, int32_t* out_accept_len,
                   int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Same operation as spec_verify_ws, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the workspace is a
 * fixed file-scope device array of SV_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends. No hipMalloc, hipFree or allocating library routine is called. Problems whose
 * spec_verify_workspace_bytes(B, D, V) exceeds SV_NOALLOC_SCRATCH_BYTES return SV_ESCRATCH and
 * enqueue nothing (32 MiB covers, e.g., B = 1024 at D = 1, V = 129280 and B = 512 at D = 7).
 * Every call on one GPU shares that GPU's scratch: calls whose stream work overlaps on one GPU
 * race and must be ordered by the caller (one stream, or events). Nothing needs clearing between
 * calls. dtype: 0 = fp32, 1 = bf16; every other argument as for spec_verify_bf16. */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_noalloc(int dtype, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const int32_t* draft_lens,
                        const float* uniforms, int B, int D, int V,
                        const float* temperature, int32_t* out_accept_len,
                        int32_t* out_tokens, hipStream_t stream);

/* Same operation, also exporting the per-row statistics the kernels computed (for tests).
 * Any export pointer may be NULL. Unused rows hold NaN / -1.
 *   row_stats   [B][2D+1][2] fp32: (max of logits/T, ln sum exp(logits/T - max)) for target
 *               rows 0..D then draft rows 0..D-1 (sampled sequences).
 *   row_argmax  [B][D+1] int32: target argmax per position (greedy sequences).
 *   logpq_x     [B][D][2] fp32: (log p_i(x_i), log q_i(x_i)) at the tested positions. */
int spec_verify_debug(int dtype, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const int32_t* draft_lens,
                      const float* uniforms, int B, int D, int V,
                      const float* temperature, int32_t* out_accept_len,
                      int32_t* out_tokens, float* row_stats, int32_t* row_argmax,
                      float* logpq_x, hipStream_t stream);

/* Threshold (relaxed) acceptance ("Accélérer Sonar par la Spéculation", section "Décodage
 * spéculatif": each prefix of the candidates is scored with a probability and the longest one
 * above an acceptance threshold is kept; the target gives one more token, sampled from its
 * logits at the first position not kept, section "Génération cible").
 *
 *   For each sampled sequence (T_b > 0) with p_i = softmax(target[b][i] / T_b): the prefix
 *   x_0..x_p is kept while sum_{i<=p} log p_i(x_i) > ln tau (its target probability is above
 *   tau); j = the first position whose prefix is not kept (L_b if all are). AL = j + 1; the
 *   tokens are x_0..x_{j-1}, then a draw from p_j by the inverse CDF in ascending token id with
 *   the uniform u[b][D] (as spec_verify's bonus draw). Draft logits are not used: no draft
 *   pointer is taken and no draft row is read. Greedy sequences (T_b = 0) follow spec_verify's
 *   argmax matching, which is this rule for any tau in [0, 1).
 *   tau: host float >= 0 (0 keeps every prefix; tau >= 1 keeps none); NaN or infinite gives
 *   SV_EINVAL. dtype: 0 = fp32, 1 = bf16. Every other argument, the layouts, the per-row error
 *   marks and the library workspace are those of spec_verify_bf16 / spec_verify_f32. */
int spec_verify_threshold(int dtype, const void* target_logits, const int32_t* draft_tokens,
                          const int32_t* draft_lens, const float* uniforms, int B, int D, int V,
                          const float* temperature, float tau, int32_t* out_accept_len,
                          int32_t* out_tokens, hipStream_t stream);

/* Saguaro draft reshaping ("Speculative Speculative Decoding - асинхронизируй это", saguaro
 * sampling: the draft's top-5 tokens get their probabilities lowered when the draft is
 * generated, so that the residual the target samples after a rejection concentrates on them;
 * the page gives no factor or formula). Reshapes draft logits in place so that softmax(l'/T) is
 * q with its top-k tokens scaled by `factor` and renormalised: for every sampled sequence
 * (T_b > 0) and position i < L_b, the k largest logits of draft row [b][i] (ties: lowest index)
 * become fp32(l + fp32(T_b * ln factor)) (ln factor rounded to fp32 on the host; bf16 rows round
 * the sum to nearest, ties to even). Draw the draft tokens from the reshaped rows and pass the
 * same rows to spec_verify: verification against the distribution the drafts came from stays
 * lossless for any factor.
 *   dtype 0 = fp32, 1 = bf16; draft_logits [B][D][V] device, updated in place; draft_lens [B]
 *   (NULL: all D) and temperature [B] device as for spec_verify. Greedy sequences, rows at
 *   positions >= L_b and sequences with an invalid length or temperature are left unchanged.
 *   factor in (0, 1]; k in [1, 8] (the page's choice is 5; k > V reshapes every token).
 * Each needed row is read once, in units; the units' candidates meet in a workspace: the
 * library-owned one of (current device, stream), allocated on first use and grown in stream
 * order like spec_verify_bf16's (refused with SV_ENOMEM under graph capture), held until
 * spec_verify_release(stream).
 * Returns SV_EINVAL (factor or k out of range, bad sizes, NULL draft_logits with D > 0 or NULL
 * temperature), SV_EDTYPE, SV_ENODEV, SV_ENOMEM or SV_EHIP, enqueueing nothing on an argument
 * error. Logits must be finite in the rows it reads. Nothing is synchronised. */
int spec_verify_saguaro_reshape(int dtype, void* draft_logits, const int32_t* draft_lens,
                                const float* temperature, int B, int D, int V, float factor,
                                int k, hipStream_t stream);

/* Bytes of device workspace spec_verify_saguaro_reshape_ws needs for shape (B, D, V) (0 on bad
 * sizes). */
size_t spec_verify_saguaro_workspace_bytes(int B, int D, int V);

/* spec_verify_saguaro_reshape with a caller-provided device workspace of at least
 * spec_verify_saguaro_workspace_bytes(B, D, V) bytes, 256-byte aligned (SV_ENOMEM otherwise;
 * NULL gives SV_EINVAL). Nothing is allocated. The workspace needs no initialisation (each call
 * writes every part it reads) and must not be used by two calls whose stream work overlaps. */
int spec_verify_saguaro_reshape_ws(int dtype, void* draft_logits, const int32_t* draft_lens,
                                   const float* temperature, int B, int D, int V, float factor,
                                   int k, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Epilogue of a verification step, on the GPU with no host synchronisation ("Accélérer Sonar
 * par la Spéculation", section "Calendrier MTP pour un jeton unique": the target's input tokens
 * are shifted and a kernel writes the newly produced tokens into their slots; section
 * "Inférence avec décodage spéculatif": the accepted count sets each sequence's next length).
 *
 *   accept_len [B]       int32, device: AL of each sequence (a spec_verify output).
 *   tokens     [B][D+1]  int32, device: the emitted tokens (a spec_verify output).
 *   input_ids  [B][W]    int32, device, updated in place: each sequence's W most recent
 *                        tokens, oldest first. The window moves AL places towards the newest
 *                        token and tokens[b][0..AL-1] fill its last AL slots (only the last W
 *                        of them when AL > W). Must not overlap accept_len, tokens or seq_len.
 *   seq_len    [B]       int32, device, updated in place: grows by AL. May be NULL.
 *
 * A sequence with AL outside [1, D+1] (AL = 0 marks a row spec_verify found invalid), or with
 * seq_len[b] < 0 or seq_len[b] + AL > 2^31 - 1, is left unchanged. Enqueued on `stream` (run
 * it on the stream of the spec_verify call whose outputs it reads); nothing is allocated or
 * synchronised. Returns SV_EINVAL for a NULL required pointer, B <= 0, D outside [0, SV_MAX_D]
 * or W <= 0 (enqueueing nothing), SV_ENODEV without a device, SV_EHIP for a failed launch. */
int spec_verify_advance(const int32_t* accept_len, const int32_t* tokens, int B, int D,
                        int32_t* input_ids, int W, int32_t* seq_len, hipStream_t stream);

/* Releases the library-owned workspaces of the plain entry points (verification and Saguaro
 * reshaping) for (current device, stream),
 * in stream order (hipFreeAsync on `stream`: the buffer is freed after the stream's earlier
 * work). Call it before destroying a stream that called spec_verify_bf16 / _f32 /
 * _threshold / _saguaro_reshape; a later call on the stream allocates again. Returns SV_OK (also when the stream
 * holds no buffer), SV_ENODEV without a device, SV_EHIP if the free fails. */
int spec_verify_release(hipStream_t stream);

/* The row launches spec_verify_bf16 / _f32 / _ws / _noalloc / _threshold make for shape
 * (B, D, V) and dtype (0 = fp32, 1 = bf16): launch s reads the rows at positions
 * [cuts[s], cuts[s + 1]) and, for s > 0, skips every row past a sequence's first rejection
 * among the earlier positions (those rows are not needed: AL and the tokens do not depend on
 * them). Writes up to max_cuts boundaries (the number of launches plus one) to the host array
 * cuts and returns the number of launches, or SV_EINVAL. For benchmarks and tests that count
 * the bytes read; spec_verify_debug reads every row in one launch. */
int spec_verify_row_stages(int dtype, int B, int D, int V, int* cuts, int max_cuts);

/* Static text for a status code. */
const char* spec_verify_strerror(int code);

/* Library ABI version (major * 100 + minor). */
int spec_verify_version(void);

/* Timing hook for benchmarks. spec_verify_profile_start(n) creates n event pairs on the current
 * device; each following row-kernel launch (any entry point, in call order; a call makes one
 * launch per stage of spec_verify_row_stages and per slice of 32767 sequences) takes one pair as
 * its own start and end stamps, until the n pairs are used. The decision kernels between stages
 * and the later kernels of a call are not timed. spec_verify_profile_stop waits for those events,
 * writes up to max_out durations in milliseconds, in launch order, to the host array out_ms (may
 * be NULL), the number of recorded launches to *n_recorded, and releases the events. Returns
 * SV_EINVAL if not started (stop) or already started (start), SV_EHIP on a runtime failure. */
int spec_verify_profile_start(int max_calls);
int spec_verify_profile_stop(float* out_ms, int max_out, int* n_recorded);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
