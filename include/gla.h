/*
 * gla.h -- C ABI of the Simple GLA library for AMD MI355X (gfx950).
 *
 * Simple GLA is the gated-linear-attention token mixer of the Laplace 3B
 * model (page "Beyond the KV cache: training and serving i14's Laplace 3B
 * linear attention model on AWS Trainium2", section "GLA mixer"). For every
 * head h a dk x dv fp32 matrix state S is decayed by a fixed per-head factor
 * lambda_h (section "Decay scheme": fixed at initialisation, not learned) and
 * receives the key/value outer product of each token; the token's output
 * reads the updated state with its query:
 *
 *     S_t = lambda_h * S_{t-1} + k_t^T v_t        o_t = scale * q_t S_t
 *
 * (k_t, q_t are 1 x dk rows, v_t and o_t are 1 x dv rows; the readout uses
 * the state after the update.)
 *
 * Prefill computes this chunkwise (same page, section "Challenge 1": inside a
 * chunk a masked, decay-weighted linear attention; across chunks a carried
 * state advanced by the decay accumulated over the chunk). Decode updates one
 * fixed-size state per sequence in place (section "Inference optimisation on
 * Trainium2": one fixed state page per sequence, read and written back at
 * every token).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to caller-owned memory, dense and
 *     row-major in the documented layout, 16-byte aligned (the workspace
 *     too; GLA_ERR_ALIGN otherwise). The library never allocates, frees or
 *     keeps a pointer after it returns.
 *   - `decay_host` is a HOST array of H floats, read during the call only.
 *     Every lambda must be finite with 0 < lambda <= 1.
 *   - `dt` is the dtype of q, k, v and o (GLA_F32 or GLA_BF16). States and
 *     initial states are always fp32.
 *   - Shapes: 1 <= H <= 64; dk and dv multiples of 16 with dk <= 128 and
 *     dv <= 256. `chunk` is the number of tokens per chunk: 0 (the library
 *     default, 64), 64 or 32; results do not depend on it beyond rounding.
 *     64 runs on the matrix cores where the shape allows, 32 always on the
 *     vector ALUs. Any other value, 128 included, returns
 *     GLA_ERR_UNSUPPORTED: no kernel here runs 128-token chunks (the
 *     Laplace 3B page's 128 matches the 128 partitions of a Trainium2
 *     on-chip buffer; on gfx950 two double-buffered 128-token tiles of q,
 *     k and v do not fit the 160 KB LDS beside the published state).
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is
 *     enqueued on it as kernel launches; no call synchronises, allocates or
 *     records a memset, so a sequence of calls may be captured into a HIP
 *     graph and replayed (the decay values and sizes are fixed at capture).
 *   - Environment, read at every call (a workspace query and the call it
 *     sizes must see the same values):
 *     GLA_TARGET_WGS (default 256, one per compute unit) is the number of
 *     workgroups below which a call splits its sequences into time
 *     segments; it changes the workspace size, never the results beyond
 *     rounding.
 *     GLA_FWD_CHAIN=1 runs a bf16 forward of a fixed batch with time
 *     segments (d_k 64 or 96, H a multiple of 8) as one chained-scan
 *     launch instead of state pass, combine and output pass; it needs a
 *     larger workspace and agrees with the default within rounding.
 *     GLA_BWD_TAIL (a fraction in [0, 0.5]; default 0.25 at dk 64, 0.1875
 *     otherwise) is the share of each sequence's chunks whose dk and dv
 *     rows the one-launch backward gives to the dq walk's workgroups;
 *     results are identical bit for bit at every share.
 *   - Arguments are validated on the host before any HIP call. On an error
 *     nothing is launched and no output is touched. A launch failure returns
 *     GLA_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP work.
 *   - Calls are stateless and re-entrant. Results are bitwise reproducible
 *     run to run (no atomics feed any output).
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 2
#define GLA_MAX_HEADS 64

typedef enum gla_status {
  GLA_OK = 0,
  GLA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  GLA_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent */
  GLA_ERR_DTYPE = 3,       /* dt is not GLA_F32 / GLA_BF16                     */
  GLA_ERR_DECAY = 4,       /* a lambda is not finite or not in (0, 1]          */
  GLA_ERR_ALIAS = 5,       /* an output overlaps an input it may not overlap   */
  GLA_ERR_UNSUPPORTED = 6, /* valid but unsupported (dk, dv, H or chunk)       */
  GLA_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required       */
  GLA_ERR_HIP = 8,         /* a HIP launch failed                              */
  GLA_ERR_ALIGN = 9,       /* a tensor pointer is not 16-byte aligned          */
  GLA_ERR_TOO_LARGE = 10,  /* needs more than GLA_NOALLOC_SCRATCH_BYTES        */
  /* not statuses: they widen the type's range to all of int, so that any
     int a caller passes is a value of the type (unknown ones well-defined) */
  GLA_STATUS_RANGE_ = 0x7fffffff,
  GLA_STATUS_RANGE_MIN_ = -0x7fffffff - 1
} gla_status;

typedef enum gla_dtype {
  GLA_F32 = 0,
  GLA_BF16 = 1,
  /* not dtypes: they widen the type's range to all of int, so that an
     unknown value passed by a caller is rejected with GLA_ERR_DTYPE, not
     undefined */
  GLA_DTYPE_RANGE_ = 0x7fffffff,
  GLA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1
} gla_dtype;

/* Activation of the output gate (gla_chunk_fwd_gated and its packed and
   decode forms): act(z) = 1 / (1 + e^-z) for sigmoid, z / (1 + e^-z) for
   SiLU. */
typedef enum gla_gate {
  GLA_GATE_SIGMOID = 1,
  GLA_GATE_SILU = 2,
  /* not gates: they widen the type's range to all of int (see gla_dtype) */
  GLA_GATE_RANGE_ = 0x7fffffff,
  GLA_GATE_RANGE_MIN_ = -0x7fffffff - 1
} gla_gate;

/* ABI version of the loaded library (GLA_ABI_VERSION at build time). */
int gla_abi_version(void);

/* Static, human-readable text for a status code. */
const char *gla_status_str(gla_status s);

/*
 * Chunked forward (prefill / training forward) of a fixed-length batch.
 *   q, k    : [B, T, H, dk]  dt
 *   v       : [B, T, H, dv]  dt
 *   s0      : [B, H, dk, dv] fp32, or NULL for zero initial states
 *   o       : [B, T, H, dv]  dt, written (not read)
 *   s_final : [B, H, dk, dv] fp32, or NULL to skip; may equal s0 (in place),
 *             otherwise must not overlap any other argument
 *   workspace: device scratch of at least gla_chunk_fwd_workspace_bytes()
 *             bytes (NULL allowed when that is 0); its contents on entry
 *             are ignored, and it must not be used by other work on other
 *             streams while the call's kernels run.
 * bf16 with dk = 96, 64 or 128 and dv a multiple of 64 runs on the matrix
 * cores (64-token chunks); fp32, other head sizes and chunk = 32 run on the vector
 * ALUs (fp32 arithmetic, 32- or 64-token chunks).
 * T = 0 is valid: o is untouched and s_final receives s0 (or zeros).
 * B * T must stay below 2^31 tokens.
 */
size_t gla_chunk_fwd_workspace_bytes(gla_dtype dt, int B, int T, int H, int dk,
                                     int dv, int chunk);
gla_status gla_chunk_fwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                         int chunk, const void *q, const void *k,
                         const void *v, const float *decay_host, float scale,
                         const float *s0, void *o, float *s_final,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Chunked forward of N packed variable-length sequences. Sequence n owns
 * tokens [cu_seqlens[n], cu_seqlens[n+1]) of the packed arrays; chunks never
 * cross a sequence boundary and each sequence starts from its own state.
 *   cu_seqlens: [N + 1] int32 DEVICE array, cu[0] = 0, non-decreasing,
 *               cu[N] = total_T. (It lives on the device, so it is not
 *               validated; values outside [0, total_T] are clamped into that
 *               range so that no access leaves the arrays, but the results
 *               are then meaningless.)
 *   q, k    : [total_T, H, dk]  dt        v, o : [total_T, H, dv]  dt
 *   s0      : [N, H, dk, dv] fp32 or NULL; s_final : [N, H, dk, dv] or NULL
 *   workspace: as for gla_chunk_fwd, at least
 *             gla_chunk_fwd_varlen_workspace_bytes() bytes. With more than
 *             one sequence it is never 0: it holds at least the dispatch
 *             order (the sequences sorted longest first, computed on the
 *             device), and, when there are too few sequences to fill the
 *             GPU, the time segments and their states.
 * A zero-length sequence is valid: its s_final is s0[n] (or zeros).
 */
size_t gla_chunk_fwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T,
                                            int H, int dk, int dv, int chunk);
gla_status gla_chunk_fwd_varlen(gla_dtype dt, int N, int total_T, int H,
                                int dk, int dv, int chunk,
                                const int32_t *cu_seqlens, const void *q,
                                const void *k, const void *v,
                                const float *decay_host, float scale,
                                const float *s0, void *o, float *s_final,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * The mixer's output gate (Laplace 3B / Trainium2 page, section "QKVG
 * projection": the fused input projection yields a gate vector g_t beside
 * q_t, k_t and v_t, and g_t acts on the mixer's output). The page names no
 * activation; the caller chooses sigmoid or SiLU:
 *     y_t = o_t * act(g_t)     (elementwise; o_t the ungated output above)
 * applied in fp32 to each output value before its single rounding to dt.
 *   g   : [B, T, H, dv] dt (gla_chunk_fwd_gated), [total_T, H, dv] dt
 *         (gla_chunk_fwd_varlen_gated), [N, H, dv] dt (gla_decode_step_gated):
 *         o's layout; read only, and o must not overlap it
 *   gate: GLA_GATE_SIGMOID or GLA_GATE_SILU (else GLA_ERR_UNSUPPORTED)
 * Every other argument, check, workspace size (the ungated call's
 * *_workspace_bytes query) and state result is that of the ungated call:
 * the gate changes the outputs only, never the recurrence's state.
 */
gla_status gla_chunk_fwd_gated(gla_dtype dt, int B, int T, int H, int dk, int dv,
                               int chunk, const void *q, const void *k, const void *v,
                               const void *g, gla_gate gate, const float *decay_host,
                               float scale, const float *s0, void *o, float *s_final,
                               void *workspace, size_t workspace_bytes, void *stream);
gla_status gla_chunk_fwd_varlen_gated(gla_dtype dt, int N, int total_T, int H, int dk, int dv,
                                      int chunk, const int32_t *cu_seqlens, const void *q,
                                      const void *k, const void *v, const void *g,
                                      gla_gate gate, const float *decay_host, float scale,
                                      const float *s0, void *o, float *s_final,
                                      void *workspace, size_t workspace_bytes, void *stream);
gla_status gla_decode_step_gated(gla_dtype dt, int N, int H, int dk, int dv, const void *q,
                                 const void *k, const void *v, const void *g, gla_gate gate,
                                 const float *decay_host, float scale, float *state, void *o,
                                 void *stream);

/*
 * gla_chunk_fwd_varlen for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, checks and results (bitwise) as
 * gla_chunk_fwd_varlen, without the workspace: the scratch comes from a
 * fixed array of GLA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's array (hipGetSymbolAddress, with that
 * device made current for the lookup). The device is the one `stream`
 * belongs to (the current device for the null stream).
 *   - A call whose plan needs more scratch than the array holds returns
 *     GLA_ERR_TOO_LARGE and launches nothing. At H = 16, dk = 96, dv = 192
 *     every packed batch fits (the largest plan, 7 long sequences cut into
 *     22 time segments, needs about 26 MB); gla_chunk_fwd_varlen_workspace_
 *     bytes() gives the need of any other shape.
 *   - Every call on a GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from different threads)
 *     race and must not be issued. Calls in sequence on one stream are
 *     safe. No byte of the array needs to start at zero: each call writes
 *     every scratch value it reads.
 */
#define GLA_NOALLOC_SCRATCH_BYTES (32u << 20)
gla_status gla_chunk_fwd_varlen_noalloc(gla_dtype dt, int N, int total_T, int H,
                                        int dk, int dv, int chunk,
                                        const int32_t *cu_seqlens, const void *q,
                                        const void *k, const void *v,
                                        const float *decay_host, float scale,
                                        const float *s0, void *o, float *s_final,
                                        void *stream);

/*
 * Backward of gla_chunk_fwd (training): given dL/do and optionally
 * dL/dS_final, the gradients with respect to q, k, v and the initial state.
 * The chain rule through the recurrence (Laplace 3B / Trainium2 page,
 * sections "GLA mixer" and "Challenge 3": training differentiates through
 * every sequential state update), with G_t = dL/dS_t:
 *   G_t = lambda G_{t+1} + scale q_t^T dO_t   (dL/dS_final enters at t = T-1)
 *   dq_t = scale dO_t S_t^T   dk_t = v_t G_t^T   dv_t = k_t G_t   dS0 = lambda G_0
 * The decays are fixed, so there is no decay gradient.
 *   q, k, v, s0, scale, decay_host : exactly as given to the forward
 *   dout     : [B, T, H, dv] dt (dL/do)
 *   ds_final : [B, H, dk, dv] fp32 or NULL (zero)
 *   dq, dk_grad : [B, T, H, dk] dt, written    dv_grad : [B, T, H, dv] dt, written
 *   ds0      : [B, H, dk, dv] fp32 or NULL to skip
 *   workspace: at least gla_chunk_bwd_workspace_bytes() bytes (fp32 partial
 *              sums of dq and dk over dv tiles and, when sequences are split
 *              into time segments, the segments' incoming states and carried
 *              gradients); NULL allowed when that is 0.
 * Shapes, dtypes and chunk as for gla_chunk_fwd: bf16 with dk = 64, 96 or
 * 128 and dv a multiple of 64 runs on the matrix cores; fp32, other head
 * sizes and chunk = 32 run on the vector ALUs (fp32 arithmetic). The workspace is
 * 0 when one workgroup covers all of dv (bf16 with dv = 64, 128 or 192 at
 * dk = 64 or 96, dv = 64 or 128 at dk = 128) and no sequence is cut into
 * time segments. Checks as for
 * gla_chunk_fwd; no output may overlap an input or another output. T = 0 is
 * valid: ds0 receives ds_final (or zeros).
 */
size_t gla_chunk_bwd_workspace_bytes(gla_dtype dt, int B, int T, int H, int dk,
                                     int dv, int chunk);
gla_status gla_chunk_bwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                         int chunk, const void *q, const void *k, const void *v,
                         const float *decay_host, float scale, const float *s0,
                         const void *dout, const float *ds_final, void *dq,
                         void *dk_grad, void *dv_grad, float *ds0, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Backward of gla_chunk_fwd_varlen: the arguments of gla_chunk_bwd in the
 * packed layout of gla_chunk_fwd_varlen (q, k, dq, dk_grad [total_T, H, dk];
 * v, dout, dv_grad [total_T, H, dv]; s0, ds_final, ds0 [N, H, dk, dv];
 * cu_seqlens [N + 1] int32 on the device, as for the forward). Same support,
 * checks and workspace rules; a zero-length sequence passes its ds_final
 * (or zeros) straight to ds0.
 */
size_t gla_chunk_bwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T, int H,
                                            int dk, int dv, int chunk);
gla_status gla_chunk_bwd_varlen(gla_dtype dt, int N, int total_T, int H, int dk,
                                int dv, int chunk, const int32_t *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const float *decay_host, float scale, const float *s0,
                                const void *dout, const float *ds_final, void *dq,
                                void *dk_grad, void *dv_grad, float *ds0, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Normalised causal linear attention (the tutorial page on RNNs without
 * recurrence, section 6.1, with the 1e-6 denominator term of the module in
 * its section 6.2). Per head, with the feature map phi = ReLU and no decay:
 *   S_t = S_{t-1} + phi(k_t)^T v_t        z_t = z_{t-1} + phi(k_t)
 *   o_t = phi(q_t) S_t / (phi(q_t) . z_t + 1e-6)
 * computed chunkwise by the same kernels as gla_chunk_fwd at lambda = 1
 * (the denominator is the readout of a value column of ones).
 *   q, k    : [B, T, H, dk] dt, raw (phi is applied inside)
 *   v, o    : [B, T, H, dv] dt (o written)
 *   s0, z0  : [B, H, dk, dv] / [B, H, dk] fp32 running sums carried in from
 *             earlier tokens, or NULL for zeros
 *   s_final, z_final : the sums after the last token, or NULL to skip
 *   workspace: device scratch of gla_linear_attn_fwd_workspace_bytes()
 *             bytes (0 unless the batch is split into time segments).
 * Shapes, dtypes and chunk as for gla_chunk_fwd (the matrix-core path for
 * bf16 with dk = 96, 64 or 128 and dv a multiple of 64). Every output must be disjoint
 * from every other argument (no in-place final sums: GLA_ERR_ALIAS).
 * T = 0 copies s0 and z0 (or zeros) to the final sums.
 */
size_t gla_linear_attn_fwd_workspace_bytes(gla_dtype dt, int B, int T, int H,
                                           int dk, int dv, int chunk);
gla_status gla_linear_attn_fwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                               int chunk, const void *q, const void *k, const void *v,
                               const float *s0, const float *z0, void *o,
                               float *s_final, float *z_final, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * gla_linear_attn_fwd over N packed variable-length sequences bounded by
 * cu_seqlens (as for gla_chunk_fwd_varlen): q, k [total_T, H, dk], v, o
 * [total_T, H, dv]; s0, s_final [N, H, dk, dv]; z0, z_final [N, H, dk].
 * Workspace: gla_linear_attn_fwd_varlen_workspace_bytes() bytes (never 0
 * for N > 1: it holds the dispatch order). Same checks as
 * gla_linear_attn_fwd; a zero-length sequence copies its s0 and z0 (or
 * zeros) to the final sums.
 */
size_t gla_linear_attn_fwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T,
                                                  int H, int dk, int dv, int chunk);
gla_status gla_linear_attn_fwd_varlen(gla_dtype dt, int N, int total_T, int H, int dk,
                                      int dv, int chunk, const int32_t *cu_seqlens,
                                      const void *q, const void *k, const void *v,
                                      const float *s0, const float *z0, void *o,
                                      float *s_final, float *z_final, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * One decode step of the normalised linear attention for N sequences (one
 * token each), continuing from the sums gla_linear_attn_fwd returns:
 *   S += phi(k)^T v,   z += phi(k),   o = phi(q) S / (phi(q) . z + 1e-6)
 *   q, k : [N, H, dk] dt   v, o : [N, H, dv] dt (o written)
 *   state: [N, H, dk, dv] fp32 and z: [N, H, dk] fp32, both updated in place
 * Checks as for gla_decode_step; o, state and z overlap nothing else.
 */
gla_status gla_linear_attn_decode_step(gla_dtype dt, int N, int H, int dk, int dv,
                                       const void *q, const void *k, const void *v,
                                       float *state, float *z, void *o, void *stream);

/*
 * The short causal convolution in front of the mixer (Laplace 3B / Trainium2
 * page, section on normalisation and convolution): every channel passes
 * through a causal Conv1d of width 4, then SiLU:
 *   z_t[c] = bias[c] + sum_{j<4} w[c][j] x_{t-3+j}[c]     y_t[c] = z / (1 + e^-z)
 *   x, y       : [B, T, D] dt (y written)
 *   w          : [D, 4] fp32 DEVICE array, tap 3 on the current token
 *   bias       : [D] fp32 device array or NULL (zero)
 *   window_in  : [B, 4, D] fp32 or NULL: the 4 most recent inputs before x,
 *                oldest first (zeros when NULL)
 *   window_out : [B, 4, D] fp32 or NULL: the 4 most recent inputs after x
 *                (the decode window to continue from); may not overlap
 *                window_in
 * D must be a multiple of 8 (GLA_ERR_UNSUPPORTED otherwise); 16-byte
 * alignment for x, y, w and the windows, 4 bytes for bias; y and
 * window_out may not overlap any input. T = 0 copies window_in (or zeros)
 * to window_out.
 */
gla_status gla_short_conv_fwd(gla_dtype dt, int B, int T, int D, const void *x,
                              const float *w, const float *bias, const float *window_in,
                              void *y, float *window_out, void *stream);

/*
 * One decode step of the short convolution for N sequences (one token
 * each): window [N, 4, D] fp32 shifts by one token in place (the oldest
 * input drops out, x[n] enters last) and y[n] = SiLU(bias + sum_j w[:, j]
 * window[n, j]). x, y : [N, D] dt. Checks as for gla_short_conv_fwd.
 */
gla_status gla_short_conv_decode_step(gla_dtype dt, int N, int D, const void *x,
                                      const float *w, const float *bias, float *window,
                                      void *y, void *stream);

/*
 * One decode step for N independent sequences (one token each):
 *   state[n,h] <- lambda_h * state[n,h] + k[n,h]^T v[n,h]    (in place)
 *   o[n,h]     <- scale * q[n,h] state[n,h]                  (after update)
 *   q, k  : [N, H, dk] dt      v : [N, H, dv] dt      o : [N, H, dv] dt
 *   state : [N, H, dk, dv] fp32, read and written in place; must not
 *           overlap q, k, v or o.
 * N = 0 is valid and does nothing.
 */
gla_status gla_decode_step(gla_dtype dt, int N, int H, int dk, int dv,
                           const void *q, const void *k, const void *v,
                           const float *decay_host, float scale, float *state,
                           void *o, void *stream);

/*
 * One decode step for N sequences whose states live in a pool of fixed,
 * per-sequence pages (a state page per sequence that stays in place across
 * steps, and batches padded to fixed widths: the inference section of the
 * Laplace 3B / Trainium2 page). Row n of q, k, v and o belongs to the
 * sequence whose state is pool entry slots[n]:
 *   state_pool[s,h] <- lambda_h * state_pool[s,h] + k[n,h]^T v[n,h]
 *   o[n,h]          <- scale * q[n,h] state_pool[s,h]     with s = slots[n]
 *   slots      : [N] int32 DEVICE array. A value outside [0, pool_size)
 *                marks a padding row: its o row is written as zeros and no
 *                state is read or written. The valid slots of one call must
 *                be distinct (two rows updating one entry race); this lives
 *                on the device and is not checked.
 *   state_pool : [pool_size, H, dk, dv] fp32, updated in place; entries no
 *                row names are not touched.
 *   q, k, v, o : as for gla_decode_step. Checks as for gla_decode_step, plus
 *                pool_size >= 1, slots non-NULL and 4-byte aligned, and no
 *                overlap of state_pool or o with any other argument.
 * N = 0 is valid and does nothing.
 */
gla_status gla_decode_step_pool(gla_dtype dt, int N, int H, int dk, int dv,
                                const void *q, const void *k, const void *v,
                                const float *decay_host, float scale,
                                const int32_t *slots, int pool_size,
                                float *state_pool, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
