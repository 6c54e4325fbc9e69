/*
 * la.h -- C ABI of liblinattn, causal linear attention run as the unified
 * recurrence on MI355X (gfx950).
 *
 * The operation (per batch b, head h; "Module 22: Linear & Recurrent
 * Attention", section "Interactive Exploration: The One Recurrence Behind
 * Them All", with the feature map and normaliser of section "The Math:
 * Linear Attention"):
 *
 *     S_t = A_t S_{t-1} + phi(k_t)^T v_t          S is d_k x d_v, fp32
 *     z_t = A_t z_{t-1} + phi(k_t)                 (only when normalising)
 *     o_t = phi(q_t) S_t   [ / (phi(q_t) . z_t) ]  read after the update
 *
 * with the gate A_t = 1 (linear attention), a per-head scalar gamma
 * (retention, section "Retention: Add a Decay to the State"), a diagonal
 * d_k x d_k gate exp(log_alpha_t) (gated linear attention, the
 * input-dependent row of the gate table) or an input-dependent scalar gate
 * exp(log_alpha_t) I per token and head (the same row with one gate value,
 * as in the section's scalar demonstration gate).  Under a gate, z is decayed by the
 * same A_t as S.  There is no epsilon in the divide.
 *
 * la_chunk_fwd computes a whole prefill in the chunkwise-parallel form
 * ("Module 22", section "The Three Faces of Retention"; "linear_sparse_
 * attention.py", linear_attn_chunkwise, including a ragged last chunk):
 * inside a chunk the in-chunk causal (decay-masked) scores times V plus the
 * query times the carried state; between chunks the carried state update.
 * la_decode_step folds one new token per (b,h) into a resident state, the
 * recurrent face ("Module 22", incremental decoding with a running state;
 * "causal linear attention as an RNN").
 *
 * Conventions shared by every entry point
 *  - Layouts are dense and row-major with the last index fastest:
 *      q, k  [B,H,L,dk]   v, out [B,H,L,dv]   (dtype of la_desc.dtype)
 *      S     [B,H,dk,dv]  fp32, rows indexed by the key channel
 *      z     [B,H,dk]     fp32
 *      log_alpha [B,H,L,dk] (DIAG) or [B,H,L] (SCALAR) fp32 natural-log
 *                gates, every value <= 0
 *  - Device pointers are device (HBM) addresses; `gamma` is a host array.
 *  - The caller owns every buffer.  The library never allocates device
 *    memory, frees or synchronises; work is enqueued on `stream` (a
 *    hipStream_t; NULL = the null stream) and runs asynchronously.
 *  - Validation runs on the host before anything is enqueued; on any error
 *    nothing is enqueued, the status is returned and a message is available
 *    from la_last_error_message() (thread-local).  No C++ exception crosses
 *    the ABI.
 *  - Device pointers must be 16-byte aligned.
 *  - log_alpha is read on the device and is not validated; values > 0 are
 *    outside the contract.
 */
#ifndef LINATTN_LA_H
#define LINATTN_LA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_VERSION 1
#define LA_MAX_GAMMA_HEADS 256 /* heads supported with LA_GATE_GAMMA */

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_INVALID = 1,     /* bad argument (checked on the host)         */
    LA_ERR_UNSUPPORTED = 2, /* valid, but outside the built kernel shapes */
    LA_ERR_HIP = 3          /* the HIP runtime reported an error          */
} la_status;

typedef enum la_gate_mode {
    LA_GATE_NONE = 0,  /* A_t = 1                                          */
    LA_GATE_GAMMA = 1, /* A_t = gamma[h]; host float[H], 0 <= gamma <= 1     */
    LA_GATE_DIAG = 2,  /* A_t = diag(exp(log_alpha[b,h,t,:])); device fp32   */
    LA_GATE_SCALAR = 3 /* A_t = exp(log_alpha[b,h,t]) I; device fp32, one
                          gate per token and head                          */
} la_gate_mode;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef enum la_phi {
    LA_PHI_IDENTITY = 0, /* phi(x) = x                                      */
    LA_PHI_ELU1 = 1      /* phi(x) = elu(x) + 1: x + 1 if x > 0, else exp(x) */
} la_phi;

typedef struct la_desc {
    int B, H;      /* batch, heads (>= 1)                                   */
    int L;         /* tokens per sequence (>= 1); must be 1 for decode      */
    int dk, dv;    /* key and value width                                    */
    int dtype;     /* la_dtype of q, k, v and out (states are always fp32)  */
    int phi;       /* la_phi, applied to q and k only                        */
    int normalize; /* 1: divide by phi(q).z and carry z; 0: no z at all     */
    int segments;  /* prefill: sequence segments per (b,h) that run in
                      parallel and are joined by a state scan; 0 = choose
                      automatically (about 256 workgroups in all, at least
                      4 chunks a segment), otherwise 1..ceil(L/chunk)      */
} la_desc;

/*
 * Supported kernel shapes (else LA_ERR_UNSUPPORTED):
 *   dk == dv, dk in {16, 32, 64, 128}; chunk a multiple of 16 in [16, 64],
 *   or in [80, 128] for bf16 at dk <= 64 and fp32 at dk <= 32 (the
 *   128-token tile of the in-chunk products fits the LDS there only).
 *   Chunks shorter than their tile (48; 80 to 112) run in the next tile
 *   up with its later tokens masked.
 *   dk != dv: (dk, dv) = (64, 128) or (128, 64), for the bf16 prefill
 *   (la_chunk_fwd, its group-norm, no-alloc and packed-sequence forms;
 *   chunk <= 64) and for la_decode_step in either type; the backward, the
 *   training forward and the delta rule need dk == dv.
 *   LA_F32 runs fp32 matrix cores (no bf16 rounding); LA_BF16 runs bf16
 *   matrix cores with fp32 accumulation and fp32 states, which needs
 *   dk >= 32 (la_decode_step runs no matrix cores and takes bf16 at every
 *   dk; la_delta_decode_step is built for bf16 at dk >= 32).
 *   LA_GATE_GAMMA needs H <= LA_MAX_GAMMA_HEADS.
 *   LA_GATE_DIAG / LA_GATE_SCALAR, prefill (la_chunk_fwd and its
 *   variants): the in-chunk form factorises the decay around a reference
 *   inside the chunk.  A chunk whose log-gates would push those factors
 *   past the fp32 range (a channel's log-gate sum over a wave's share of the
 *   chunk below about -83 / (waves per half chunk)) is recomputed as
 *   sequential 16-token sub-chunks, each factorised around its eighth
 *   token, with every factor applied to the state at most one.  The result
 *   stays exact (to rounding) while every 8 consecutive log-gates of a
 *   channel sum to more than about -83, e.g. log_alpha >= -10 per token.
 *   la_chunk_bwd factorises around the chunk middle only: the per-channel
 *   log-gate sum over any half chunk (32 tokens) must stay above about -83.
 */

/*
 * la_chunk_fwd -- chunkwise-parallel prefill of L tokens per (b,h).
 *   d                  shape, dtype, phi, normalize, segments
 *   q, k, v            device, [B,H,L,dk|dv] of d->dtype, read only
 *   gate_mode          la_gate_mode
 *   gamma_or_log_alpha NONE: ignored (may be NULL); GAMMA: host float[H];
 *                      DIAG: device float[B,H,L,dk]; SCALAR: device
 *                      float[B,H,L]
 *   S0, z0             device fp32 initial state [B,H,dk,dv] and [B,H,dk];
 *                      NULL = zeros.  z0 must be NULL unless normalize.
 *   chunk              chunk length C (see supported shapes)
 *   out                device [B,H,L,dv] of d->dtype, written
 *   S_final, z_final   device fp32 final state / normaliser, or NULL (not
 *                      returned).  They may alias S0 / z0 (in-place
 *                      resumption).  z_final must be NULL unless normalize.
 *   workspace          device scratch of at least
 *                      la_chunk_fwd_workspace_bytes(d, chunk) bytes, 16-byte
 *                      aligned; contents are clobbered
 *   stream             hipStream_t
 */
la_status la_chunk_fwd(const la_desc* d, const void* q, const void* k,
                       const void* v, int gate_mode,
                       const float* gamma_or_log_alpha, const float* S0,
                       const float* z0, int chunk, void* out, float* S_final,
                       float* z_final, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * la_chunk_fwd_varlen -- the same prefill over B packed sequences of
 * different lengths that share each head's token axis, each with its own
 * initial and final state (the batched prefill before recurrent decoding:
 * "Module 22", incremental decoding with a running state; the S_final of
 * each sequence is the state la_decode_step continues from).
 *   d            d->B = number of sequences, d->L = T = total tokens;
 *                d->segments as for la_chunk_fwd, counted for max_seqlen
 *   cu_seqlens   device int32 [B+1]: sequence n owns tokens
 *                [cu_seqlens[n], cu_seqlens[n+1]) of every head; the
 *                caller guarantees 0 = cu[0] <= cu[1] <= ... <= cu[B] <= T
 *                and every length <= max_seqlen (device data, not
 *                validated; the kernels clamp offsets to [0, T], so a
 *                violation gives wrong values but no access outside the
 *                tensors).  Empty sequences are allowed (S_final = S0).
 *   max_seqlen   host int, 1 <= max_seqlen <= T: the longest sequence
 *   q, k         device [H,T,dk] (a [1,H,T,dk] tensor) of d->dtype
 *   v, out       device [H,T,dv]
 *   log_alpha    DIAG: device fp32 [H,T,dk]; SCALAR: [H,T]
 *   S0, S_final  device fp32 [B,H,dk,dv] per sequence (NULL as before)
 *   z0, z_final  device fp32 [B,H,dk]
 *   workspace    la_chunk_fwd_varlen_workspace_bytes(d, max_seqlen, chunk)
 *                bytes, 16-byte aligned, never NULL: besides the segment
 *                slots it holds the launch order of the sequences (longest
 *                first, computed on the device; the order affects only
 *                the scheduling, never a result)
 * Everything else as for la_chunk_fwd.
 */
la_status la_chunk_fwd_varlen(const la_desc* d, const int* cu_seqlens,
                              int max_seqlen, const void* q, const void* k,
                              const void* v, int gate_mode,
                              const float* gamma_or_log_alpha,
                              const float* S0, const float* z0, int chunk,
                              void* out, float* S_final, float* z_final,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* Workspace bytes of la_chunk_fwd_varlen (at least 16; 0 if the arguments
 * are invalid). */
size_t la_chunk_fwd_varlen_workspace_bytes(const la_desc* d, int max_seqlen,
                                           int chunk);

/*
 * Output epilogue of retention (RetNet): each token's head output, after
 * the optional normaliser, is normalised over its d_v channels (group norm
 * with one group per head) and multiplied by swish of a gate tensor ("Module
 * 22", section "Retention: Add a Decay to the State", which names this
 * GroupNorm and swish gate as RetNet's stabiliser in place of a divide):
 *     y = (o - mean(o)) / sqrt(var(o) + eps) * weight + bias
 *     out = y * gate * sigmoid(gate)       (or out = y without a gate)
 * mean and var are over the d_v outputs of one token and head (biased
 * variance), computed in fp32.
 */
typedef struct la_groupnorm {
    const float* weight; /* device fp32 [H,dv], or NULL (ones)                 */
    const float* bias;   /* device fp32 [H,dv], or NULL (zeros)                */
    const void* gate;    /* device [B,H,L,dv] of d->dtype, or NULL (no gate)   */
    float eps;           /* > 0                                                 */
} la_groupnorm;

/*
 * la_chunk_fwd_groupnorm -- la_chunk_fwd with the epilogue above fused into
 * the store of each output chunk (out holds the epilogue's result; S_final
 * and z_final are unchanged).  Built for chunk 64 (LA_ERR_UNSUPPORTED for
 * other chunks).  Arguments as for la_chunk_fwd, plus gn (not NULL).
 */
la_status la_chunk_fwd_groupnorm(const la_desc* d, const void* q, const void* k,
                                 const void* v, int gate_mode,
                                 const float* gamma_or_log_alpha,
                                 const float* S0, const float* z0, int chunk,
                                 const la_groupnorm* gn, void* out,
                                 float* S_final, float* z_final,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * la_chunk_fwd_noalloc -- la_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, result and kernels as
 * la_chunk_fwd without the workspace pair: the segment states, decays and
 * normaliser parts live instead in a static device array of
 * LA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends.
 *   - Nothing is allocated: no hipMalloc, hipFree or allocating library
 *     call.  The array's device address is looked up once per device (on
 *     the first call whose stream belongs to that device) and kept.
 *   - LA_ERR_UNSUPPORTED when the shape's workspace
 *     (la_chunk_fwd_workspace_bytes) exceeds LA_NOALLOC_SCRATCH_BYTES; the
 *     automatic segment choice needs at most about 34 MB at d = 128.
 *   - Every call on one GPU shares that GPU's array, and the array keeps
 *     the last call's contents (every slot a call reads it has written
 *     first, so nothing needs clearing).  Calls that overlap in time on one
 *     GPU (different streams, or different host threads) race on it and
 *     give wrong results: serialise them.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
la_status la_chunk_fwd_noalloc(const la_desc* d, const void* q, const void* k,
                               const void* v, int gate_mode,
                               const float* gamma_or_log_alpha,
                               const float* S0, const float* z0, int chunk,
                               void* out, float* S_final, float* z_final,
                               void* stream);

/* Bytes of device workspace la_chunk_fwd needs for this shape: the segment
 * states, their decays and normaliser parts (several segments only) and one
 * int32 per segment (under a vector gate, whether the segment was
 * recomputed in sub-chunks).  Returns 0 for an invalid descriptor. */
size_t la_chunk_fwd_workspace_bytes(const la_desc* d, int chunk);

/* Number of segments la_chunk_fwd will run per (b,h) for this shape. */
int la_chunk_fwd_segments(const la_desc* d, int chunk);

/*
 * la_chunk_bwd -- gradients of a prefill (the reverse-mode derivative of
 * la_chunk_fwd without the normaliser) for the loss
 *     sum(dout * out) + sum(dS_final * S_final).
 * The derivative of the recurrence written out per chunk: the states before
 * every chunk are recomputed, the state gradient G runs the same recurrence
 * from the end (G_{t-1} = A_t G_t + phi(q_t)^T dout_t), and each chunk then
 * forms its gradients from its own tokens, the state before it and G after
 * it ("Module 22: Linear & Recurrent Attention", sections "The Three Faces
 * of Retention" and "The One Recurrence Behind Them All" for the forward
 * it differentiates).  The chunk length is the library's own
 * (la_chunk_bwd_chunk); the result does not depend on it beyond rounding.
 *   d                  as for la_chunk_fwd; normalize must be 0
 *                      (LA_ERR_UNSUPPORTED otherwise)
 *   q, k, v            device, [B,H,L,dk|dv] of d->dtype, the forward inputs
 *   dout               device [B,H,L,dv] of d->dtype, gradient of out
 *   gate_mode, gamma_or_log_alpha   as for la_chunk_fwd
 *   S0                 device fp32 [B,H,dk,dv] forward initial state, or NULL
 *   dS_final           device fp32 [B,H,dk,dv] gradient of S_final, or NULL
 *   states             the boundary states la_chunk_fwd_train wrote for
 *                      these inputs, or NULL (recomputed here)
 *   dq, dk, dv         device [B,H,L,dk|dv] of d->dtype, written: gradients
 *                      of the raw q, k (through phi) and v
 *   dlog_alpha         DIAG: device fp32 [B,H,L,dk], SCALAR: [B,H,L],
 *                      written; must be NULL for the other gates (gamma
 *                      gets no gradient)
 *   dS0                device fp32 [B,H,dk,dv] gradient of S0, written, or
 *                      NULL (not returned)
 *   workspace          device scratch of at least
 *                      la_chunk_bwd_workspace_bytes(d) bytes; clobbered
 *   stream             hipStream_t
 * Outputs must not alias inputs.
 */
la_status la_chunk_bwd(const la_desc* d, const void* q, const void* k,
                       const void* v, const void* dout, int gate_mode,
                       const float* gamma_or_log_alpha, const float* S0,
                       const float* dS_final, const void* states, void* dq,
                       void* dk, void* dv, float* dlog_alpha, float* dS0,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_chunk_fwd_train -- la_chunk_fwd (no normaliser, chunk
 * la_chunk_bwd_chunk(d)) that also leaves behind, in `states`, the state
 * before every chunk and the final state in the element type of q/k/v
 * ([B,H,ceil(L/C)+1,dk,dv], row-major), which la_chunk_bwd then takes
 * instead of recomputing them.
 *   states, states_bytes   device buffer of at least
 *                          la_chunk_train_states_bytes(d) bytes, written
 *   workspace              la_chunk_fwd_workspace_bytes(d, la_chunk_bwd_chunk(d))
 * Other arguments as for la_chunk_fwd (z0/z_final absent).
 */
la_status la_chunk_fwd_train(const la_desc* d, const void* q, const void* k,
                             const void* v, int gate_mode,
                             const float* gamma_or_log_alpha, const float* S0,
                             void* out, float* S_final, void* states,
                             size_t states_bytes, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the boundary states la_chunk_fwd_train writes (0 if invalid). */
size_t la_chunk_train_states_bytes(const la_desc* d);

/* Bytes of device workspace la_chunk_bwd needs: the state before each
 * chunk and the final state in the element type of q/k/v
 * (B*H*(ceil(L/C)+1)*dk*dv elements) plus the fp32 segment slots.
 * Returns 0 for an invalid descriptor. */
size_t la_chunk_bwd_workspace_bytes(const la_desc* d);

/* Chunk length C the backward uses for this shape (0 if invalid). */
int la_chunk_bwd_chunk(const la_desc* d);

/*
 * la_decode_step -- fold one token per (b,h) into the resident state.
 *   d          shape with d->L == 1 (B = sequences, H = heads)
 *   q, k, v    device [B,H,dk|dv] of d->dtype
 *   gate_mode  la_gate_mode
 *   gate       NONE: ignored; GAMMA: host float[H]; DIAG: device fp32
 *              log-gates [B,H,dk]; SCALAR: device fp32 [B,H]
 *   S          device fp32 [B,H,dk,dv], updated in place to A S + phi(k) v^T
 *   z          device fp32 [B,H,dk], updated in place; NULL iff !normalize
 *   out        device [B,H,dv] of d->dtype: phi(q)^T S_new [/ phi(q).z_new]
 *   stream     hipStream_t
 */
la_status la_decode_step(const la_desc* d, const void* q, const void* k,
                         const void* v, int gate_mode, const float* gate,
                         float* S, float* z, void* out, void* stream);

/*
 * The delta rule (DeltaNet; "linear_sparse_attention.py", function
 * delta_rule_recurrent):
 *     S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = q_t^T S_t
 * in the [dk][dv] state orientation used throughout (the page writes the
 * transpose): each token first erases what the state returns for k_t, then
 * writes v_t there with strength beta_t.  Keys are used as given (the page's
 * function assumes the caller normalised them); there is no feature map and
 * no normaliser (d->phi must be LA_PHI_IDENTITY, d->normalize 0, else
 * LA_ERR_UNSUPPORTED).  d->segments is ignored: each (b,h) runs its chunks
 * in order.
 *
 * la_delta_fwd -- prefill, in the chunkwise form with the triangular
 * factorisation of each chunk's erase products (chunk length
 * la_delta_chunk(d)).
 *   q, k     device [B,H,L,dk] of d->dtype;  v, out  device [B,H,L,dv]
 *   beta     device fp32 [B,H,L] write strengths (not validated; the page
 *            uses beta in [0, 1])
 *   S0       device fp32 [B,H,dk,dv] or NULL (zeros)
 *   S_final  device fp32 [B,H,dk,dv] or NULL; may alias S0
 * No workspace.
 */
la_status la_delta_fwd(const la_desc* d, const void* q, const void* k,
                       const void* v, const float* beta, const float* S0,
                       void* out, float* S_final, void* stream);

/*
 * la_delta_decode_step -- one token per (b,h) folded into the resident
 * state S (device fp32 [B,H,dk,dv], updated in place); q, k, v device
 * [B,H,dk|dv] of d->dtype, beta device fp32 [B,H], out device [B,H,dv].
 * d->L must be 1.
 */
la_status la_delta_decode_step(const la_desc* d, const void* q, const void* k,
                               const void* v, const float* beta, float* S,
                               void* out, void* stream);

/* Chunk length la_delta_fwd uses for this shape (0 if invalid). */
int la_delta_chunk(const la_desc* d);

/* Static description of a status code. */
const char* la_status_string(la_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* la_last_error_message(void);

/* LA_VERSION of the built library. */
int la_version(void);

/*
 * Kernel timing for benchmarks.  Between la_profile_begin() and
 * la_profile_end() every kernel the library enqueues is bracketed by a pair
 * of HIP events recorded on the stream it is launched on.  la_profile_query
 * waits for those events and reports, for one kernel family
 * ("chunk_main", "chunk_sub", "chunk_state", "state_scan", "decode", "chunk_store",
 * "chunk_bwd", "delta_chunk", "delta_decode"), the number of
 * launches and their summed duration in milliseconds.  la_profile_begin
 * clears earlier records.  Event creation happens inside la_profile_begin /
 * the first profiled launch; not for use under graph capture.
 */
la_status la_profile_begin(void);
la_status la_profile_end(void);
la_status la_profile_query(const char* kernel, int* launches,
                           double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_LA_H */
