/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library,
 * libkda.so.
 *
 * KDA keeps, per sequence and head, a fixed-shape recurrent state
 * S (dk x dv, fp32).  Each token decays the rows of S by exp(g) (one log-decay
 * per key channel), subtracts the state's prediction for the current key
 * before writing the new value (delta rule), is read by the query after the
 * write, and the readout goes through an input-dependent sigmoid gate:
 *
 *     S   <- diag(exp(g_t)) S
 *     u   =  beta_t (v_t - S^T k_t)
 *     S   <- S + k_t u^T
 *     y_t =  sigmoid(z_t) * (scale * S^T q_t)
 *
 * Sources: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
 * section 1 rows Q04 (fixed-shape state, channel-wise decay, delta-rule
 * write), Q05 (subtract the existing prediction for the key), Q06 (log-decay
 * floor -5), Q07 (chunkwise-parallel prefill with the state passed between
 * chunks; O(1) decode), Q08 (input-dependent output gate); "Kimi K3 report
 * reveals training and systems stack", confirmed list (FlashKDA, 16-token
 * tiles).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates no device memory; calls are re-entrant.  State it
 *     keeps until the process ends, per device: one auxiliary HIP stream and a
 *     few events (created at the first kda_chunk_fwd over a long single
 *     sequence, see there), its kernels' LDS attributes, and the address of
 *     the static scratch array of kda_chunk_fwd_noalloc.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without synchronising; work forked to the auxiliary stream is
 *     joined back into `stream` before the call's last kernel.  Arguments are validated on the host
 *     before anything is launched: on any error a status code is returned and
 *     nothing is written.  A failed launch returns KDA_ERR_HIP.
 *   - Layouts are row-major and contiguous.  Element types: `dt` gives the
 *     type of q, k, v, g, beta, gate and out; the state is always fp32.
 *   - Alignment: every tensor pointer 16 bytes, except beta and grad_beta
 *     (their element size) and cu_seqlens / accepted (4 bytes); workspaces
 *     and forward records 256 bytes.  A pointer below its alignment returns
 *     KDA_ERR_MISALIGNED, checked after the other arguments.  Tensors from a
 *     device allocator, and views of them at whole-token offsets, meet it.
 *   - Values are not range-checked on the device.  Documented preconditions:
 *     beta in [0, 1]; for the chunked forward g must be finite with
 *     g >= -5 (KDA_G_MIN), which bounds the reciprocal of the cumulative decay
 *     inside a 16-token subtile by exp(80) so the subtile products stay in the
 *     bf16/fp32 range ("Kimi K3 second-pass study ledger", section 1 row Q06).
 *     The decode step has no lower bound (g = -inf gives a decay of 0).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_G_MIN (-5.0f)

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL                 */
    KDA_ERR_BAD_SHAPE = 2,          /* negative/zero size, B > 1 with cu_seqlens  */
    KDA_ERR_BAD_DTYPE = 3,          /* dt is not a kda_dtype value                */
    KDA_ERR_UNSUPPORTED = 4,        /* (dt, dk, dv, chunk) outside the supported set, or
                                       more than 2^31 - 1 (chunk slot, head) pairs */
    KDA_ERR_WORKSPACE_TOO_SMALL = 5,/* workspace_bytes below the required size    */
    KDA_ERR_HIP = 6,                /* a HIP launch or runtime call failed        */
    KDA_ERR_MISALIGNED = 7,         /* a pointer below its required alignment     */
    KDA_ERR_SCRATCH_LIMIT = 8       /* kda_chunk_fwd_noalloc: the sizes need more
                                       than KDA_NOALLOC_SCRATCH_BYTES of scratch  */
} kda_status;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_str(kda_status s);

/* Supported (dt, dk, dv, chunk) combinations of kda_chunk_fwd:
 *   KDA_BF16, dk = dv = 128, chunk = 64 (four 16-token subtiles; bf16 matrix
 *            cores, fp32 accumulation and fp32 state)
 *   KDA_F32,  dk = dv = 16,  chunk = 16 (fp32 arithmetic throughout)
 * kda_decode_step supports both dtypes with dk = dv in {16, 128}.
 * Returns 1 if supported, 0 otherwise. */
int kda_chunk_fwd_supported(kda_dtype dt, int dk, int dv, int chunk);
int kda_decode_step_supported(kda_dtype dt, int dk, int dv);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 when none
 * is needed, (size_t)-1 for an unsupported or invalid combination).
 * `N` is the number of sequences; `varlen` is 1 when cu_seqlens will be
 * passed (an argument beyond the planned interface: the slot bound differs,
 * and cu_seqlens' contents are not known on the host).  The size depends only
 * on the arguments: with cu_seqlens the bound floor(T / 128) + N pair slots is
 * used for every head.
 * For KDA_BF16 the forward composes every two consecutive chunks of a sequence
 * into one step of the serial chunk-to-chunk pass and keeps one 164,352-byte
 * record per (pair of chunks, head): 1,284 bytes per token-head, against 1,538
 * bytes per token-head of inputs and outputs (B ceil(T / 128) H records, or
 * (floor(T / 128) + N) H with cu_seqlens; 21.5 GB for 2^20 tokens x 16 heads).
 * Calls that keep per-chunk records instead (KDA_FWD_CHUNK_RECORDS, or a
 * snapshot interval that is an odd multiple of 64) need
 * kda_chunk_fwd_records_bytes(...): one 180,736-byte record per
 * (chunk, head), 2,824 bytes per token-head (the chunk's map and readout,
 * and the intra-chunk factors the backward's gradient kernel reads). */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                     kda_dtype dt, int varlen);
size_t kda_chunk_fwd_records_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                   kda_dtype dt, int varlen);

/* Chunkwise-parallel KDA forward (prefill / training forward).
 *
 * The sequence is cut into chunks of `chunk` tokens; inside a chunk the
 * tokens are processed with dense matrix products, and the state is passed
 * recurrently from one chunk to the next ("Kimi K3 second-pass study
 * ledger", section 1 row Q07).  Chunking restarts at every sequence start;
 * the last chunk of a sequence may be partial.  The result equals the
 * token-by-token recurrence above up to rounding.
 *
 *   q, k, g  [B, T, H, dk]   dt          (g: natural-log decay, see above)
 *   v, gate  [B, T, H, dv]   dt          (gate: logits z; sigmoid applied here)
 *   beta     [B, T, H]       dt
 *   init_state  [N, H, dk, dv] fp32, or NULL for a zero initial state
 *   out         [B, T, H, dv]  dt, written (rounded to nearest even for bf16)
 *   final_state [N, H, dk, dv] fp32, or NULL (not written); it may alias
 *               init_state (in-place update of a state cache)
 *   cu_seqlens  NULL: B sequences of length T each, N must equal B.
 *               non-NULL: device int32 [N + 1], B must be 1; sequence n is
 *               tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed T.
 *               Preconditions (not checked): cu[0] = 0, non-decreasing,
 *               cu[N] = T.  Zero-length sequences are allowed; their final
 *               state equals their initial state.
 *   scale       multiplies the readout S^T q (1.0 for the plain form)
 *   workspace   device memory of at least kda_chunk_fwd_workspace_bytes(...)
 *               bytes, 256-byte aligned; contents on entry are ignored and
 *               left undefined.  May be NULL when the size is 0.
 * Overlapping calls that share a workspace race; out must not alias any input.
 *
 * Long single sequences (KDA_BF16, cu_seqlens NULL, B = 1, at least 65,536
 * tokens, final_state not NULL, no snapshots): the call runs in segments of
 * at least 32,768 tokens.  The serial part of each segment runs on the
 * auxiliary stream, starting from the fp32 state the previous segment left
 * in final_state, while `stream` prepares the next segment (when H <= 32) and
 * computes the outputs of finished ones.  The result is bitwise that of one
 * unsegmented pass; final_state is written during the call.
 * When `stream` is capturing a graph (hipStreamIsCapturing), every kernel
 * stays on `stream` instead, with the same result.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, const float *init_state,
                         void *out, float *final_state, const int32_t *cu_seqlens, int B, int T,
                         int N, int H, int dk, int dv, int chunk, float scale, kda_dtype dt,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation, arguments and results as kda_chunk_fwd, bit for bit,
 * without the workspace: it is taken from a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, which that
 * GPU holds from the first such call until the process ends.  The call
 * allocates nothing (no hipMalloc, no stream or event is created: every kernel
 * runs on `stream`, also for long single sequences).  Sizes whose workspace,
 * kda_chunk_fwd_workspace_bytes(...), exceeds KDA_NOALLOC_SCRATCH_BYTES
 * return KDA_ERR_SCRATCH_LIMIT before anything is launched.  Every call on one
 * GPU uses that GPU's one array: calls that overlap on a GPU (two streams or
 * two host threads without ordering between them) race and give undefined
 * results.  No byte of the array needs to start at zero: a call reads only
 * what it has written earlier in the same call. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const void *gate, const float *init_state,
                                 void *out, float *final_state, const int32_t *cu_seqlens, int B,
                                 int T, int N, int H, int dk, int dv, int chunk, float scale,
                                 kda_dtype dt, hipStream_t stream);

/* State snapshots for prefix caching and replay ("Kimi K3 second-pass study
 * ledger", section 1 row Q31 and section 3 Fig. 12: the serving engine keeps
 * sparse checkpoints of the fixed-size KDA state at hash-block boundaries, and
 * a cache hit resumes from such a checkpoint).
 *
 * kda_chunk_fwd_snapshots is kda_chunk_fwd plus `snapshots`: when non-NULL,
 * the fp32 state after the first m * snapshot_interval tokens of each sequence
 * is written for m = 1 .. floor(len / snapshot_interval) (a sequence whose
 * length is a multiple of the interval gets its final state as its last
 * snapshot).  snapshot_interval must be a positive multiple of `chunk`
 * (else KDA_ERR_BAD_SHAPE).  Snapshot m of sequence n goes to slot
 *     n * floor(T / interval) + m - 1                 (cu_seqlens NULL)
 *     floor(cu_seqlens[n] / interval) + n + m - 1     (cu_seqlens given)
 * of snapshots [slots, H, dk, dv] fp32, slots = kda_snapshot_slots(...);
 * slots that match no snapshot are not written.  Replaying a sequence from
 * snapshot m = kda_chunk_fwd on tokens m * interval .. with the snapshot as
 * init_state.  With snapshots NULL the call is exactly kda_chunk_fwd.  For
 * KDA_BF16 an interval that is an odd multiple of 64 tokens falls inside a
 * pair of chunks, so the call keeps per-chunk records and its workspace must
 * hold kda_chunk_fwd_records_bytes(...) bytes; multiples of 128 need only
 * kda_chunk_fwd_workspace_bytes(...).
 * kda_snapshot_slots returns (size_t)-1 for invalid sizes. */
size_t kda_snapshot_slots(int B, int T, int N, int chunk, int interval, int varlen);

kda_status kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const void *gate, const float *init_state,
                                   void *out, float *final_state, float *snapshots,
                                   int snapshot_interval, const int32_t *cu_seqlens, int B,
                                   int T, int N, int H, int dk, int dv, int chunk, float scale,
                                   kda_dtype dt, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Fused input prologue.  Bits of `prologue` in the *_ex entry points; each
 * applies one elementwise map to an input inside the kernels, so callers can
 * pass raw projections without separate passes over HBM:
 *   KDA_PRO_QK_L2NORM    q and k are divided by sqrt(sum over dk of x^2 + 1e-6)
 *                        per (token, head), in fp32
 *   KDA_PRO_BETA_SIGMOID beta holds logits; the write strength is sigmoid(beta)
 *   KDA_PRO_G_SOFTPLUS   g holds pre-activations x; the log-decay is
 *                        max(KDA_G_MIN, -softplus(x)), which always meets the
 *                        chunked forward's g >= -5 precondition
 * ("Kimi K3 second-pass study ledger", section 1 row Q06 for the -5 floor;
 * the other maps are the standard ones for these inputs.)  Other bits return
 * KDA_ERR_UNSUPPORTED. */
#define KDA_PRO_QK_L2NORM 1u
#define KDA_PRO_BETA_SIGMOID 2u
#define KDA_PRO_G_SOFTPLUS 4u

/* Forward flag for the *_ex entry point: keep one record per chunk (not per
 * pair of chunks) in the workspace, as kda_chunk_bwd_ex needs them; the
 * workspace must then hold kda_chunk_fwd_records_bytes(...) bytes.  No effect
 * for KDA_F32 (that path keeps no records). */
#define KDA_FWD_CHUNK_RECORDS 256u

/* kda_chunk_fwd_snapshots plus `flags`: the prologue bits and
 * KDA_FWD_CHUNK_RECORDS (0 = exactly that call).  Other bits return
 * KDA_ERR_UNSUPPORTED. */
kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const void *gate, const float *init_state,
                            void *out, float *final_state, float *snapshots,
                            int snapshot_interval, const int32_t *cu_seqlens, int B, int T,
                            int N, int H, int dk, int dv, int chunk, float scale, kda_dtype dt,
                            unsigned flags, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* One O(1) recurrent decode step for N independent sequences, updating the
 * state in place ("Kimi K3 second-pass study ledger", section 1 row Q07;
 * section 8 device row, fused decode): decay, prediction, correction, write,
 * read and gate in one pass over each state slice.
 *
 *   q, k, g  [N, H, dk]  dt        v, gate, out [N, H, dv]  dt
 *   beta     [N, H]      dt
 *   state    [N, H, dk, dv] fp32, read and overwritten in place
 * out must not alias the state or any input.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const void *gate, float *state, void *out, int N,
                           int H, int dk, int dv, float scale, kda_dtype dt, hipStream_t stream);

/* kda_decode_step plus the prologue bits (see KDA_PRO_*; 0 = exactly that call). */
kda_status kda_decode_step_ex(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const void *gate, float *state, void *out, int N,
                              int H, int dk, int dv, float scale, kda_dtype dt, unsigned prologue,
                              hipStream_t stream);

/* Speculative decoding: verify K draft tokens, then commit the accepted
 * prefix ("Kimi K3 plain-language guide", section 4.1: the MTP layer is tuned
 * into an EAGLE-3 draft model whose guesses the full model verifies; the KDA
 * state must then move past exactly the accepted tokens).
 *
 * kda_decode_verify runs the K tokens of each sequence, in order, on a copy of
 * its state held on chip, and leaves `state` unchanged.  Token t of sequence
 * n is row (n K + t) of the token-major inputs, i.e.
 *   q, k, g  [N, K, H, dk]   v, gate, out [N, K, H, dv]   beta [N, K, H]   dt
 *   state    [N, H, dk, dv]  fp32, read only
 *   u_out    [N, K, H, dv]   fp32, the delta-rule correction u of every token
 *                            (needed by kda_decode_commit; NULL = not written)
 * out[n, t] equals what t + 1 successive kda_decode_step calls would return
 * for that token, bit for bit.
 *
 * kda_decode_commit advances each state past its first accepted[n] tokens
 * (accepted: device int32 [N], clamped to 0 .. K; 0 leaves the state as it
 * is), from the same k and g given to the verification and its u_out:
 *     S <- diag(exp(g_t)) S + k_t u_t^T,   t = 0 .. accepted[n] - 1
 * The result equals accepted[n] successive kda_decode_step calls, bit for
 * bit, at the cost of one read and one write of the state.  `prologue` must
 * be the bits given to the verification. */
kda_status kda_decode_verify(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const void *gate, const float *state, void *out,
                             float *u_out, int N, int K, int H, int dk, int dv, float scale,
                             kda_dtype dt, unsigned prologue, hipStream_t stream);

kda_status kda_decode_commit(const void *k, const void *g, const float *u,
                             const int32_t *accepted, float *state, int N, int K, int H, int dk,
                             int dv, kda_dtype dt, unsigned prologue, hipStream_t stream);

/* Chunkwise KDA backward for training ("Kimi K3 second-pass study ledger",
 * section 1 row Q07: the chunkwise-parallel form serves training as well as
 * prefill).  Given the forward's inputs and the gradients of a loss with
 * respect to its outputs, returns the gradients with respect to every input
 * of kda_chunk_fwd (prepared inputs: no prologue):
 *
 *   q, k, g, v, gate, beta, init_state, cu_seqlens, B, T, N, H, dk, dv,
 *   chunk, scale, dt  exactly as given to kda_chunk_fwd
 *   grad_out          [B, T, H, dv] dt: dLoss/d out
 *   grad_final_state  [N, H, dk, dv] fp32: dLoss/d final_state, or NULL (zero)
 *   grad_q, grad_k, grad_g [B, T, H, dk] dt     written
 *   grad_v, grad_gate      [B, T, H, dv] dt     written (grad_gate: w.r.t. the logits)
 *   grad_beta              [B, T, H]     dt     written
 *   grad_init_state        [N, H, dk, dv] fp32  written, or NULL (not written);
 *                          it may alias grad_final_state
 * The gradient of g is the total one, through the decay of the state and
 * through every within-chunk decay factor.  Forward quantities are recomputed
 * inside the call (nothing is kept from a previous kda_chunk_fwd).
 * Supported: the same (dt, dk, dv, chunk) as kda_chunk_fwd
 * (kda_chunk_bwd_supported): KDA_BF16 with dk = dv = 128, chunk = 64
 * (gradients rounded to bf16, state gradients carried in fp32), and KDA_F32
 * with dk = dv = 16, chunk = 16.  Workspace: kda_chunk_bwd_workspace_bytes(...)
 * bytes, 256-byte aligned, contents ignored and left undefined.  Gradient
 * outputs must not alias the inputs or each other (except as stated). */
int kda_chunk_bwd_supported(kda_dtype dt, int dk, int dv, int chunk);

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                     kda_dtype dt, int varlen);

kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, const float *init_state,
                         const void *grad_out, const float *grad_final_state, void *grad_q,
                         void *grad_k, void *grad_v, void *grad_g, void *grad_beta,
                         void *grad_gate, float *grad_init_state, const int32_t *cu_seqlens,
                         int B, int T, int N, int H, int dk, int dv, int chunk, float scale,
                         kda_dtype dt, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* kda_chunk_bwd reusing the forward's work (training: forward, then backward
 * on the same inputs).  fwd_records = the workspace of a kda_chunk_fwd_ex
 * call with KDA_BF16, flags = KDA_FWD_CHUNK_RECORDS (no prologue bits) and
 * the same q, k, v, g, beta, init_state, cu_seqlens, sizes and scale, left
 * untouched since that call; fwd_records_bytes its size (at least
 * kda_chunk_fwd_records_bytes(...)).  The backward then skips recomputing every
 * chunk's entry state, and needs only kda_chunk_fwd_records_bytes(...) bytes
 * of `workspace`.  The records are consumed: their contents are undefined
 * afterwards.  fwd_records NULL = exactly kda_chunk_bwd; fwd_records with
 * KDA_F32 returns KDA_ERR_UNSUPPORTED (that path keeps no records). */
kda_status kda_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const void *gate, const float *init_state,
                            const void *grad_out, const float *grad_final_state, void *grad_q,
                            void *grad_k, void *grad_v, void *grad_g, void *grad_beta,
                            void *grad_gate, float *grad_init_state, const int32_t *cu_seqlens,
                            int B, int T, int N, int H, int dk, int dv, int chunk, float scale,
                            kda_dtype dt, void *fwd_records, size_t fwd_records_bytes,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
