/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA / CKDA gated delta-rule library.
 *
 * The operation (per batch b and head h, state S of d_k x d_v, fp32):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 * The update is the real form of the recurrence on the SFDA page ("Resumen
 * Tecnico: Atencion Delta de Fourier Semidirecta (SFDA)", section
 * "Arquitectura Central", with the phases at zero, which recovers KDA) and of
 * the Gated DeltaNet-2 page (section 1, erase and write gates tied to the
 * scalar beta).  Complex KDA ("Complex KDA" summary, section "Complex KDA
 * (CKDA) Mimarisi") widens the ranges to alpha in [-1, 1] per key channel and
 * beta in [0, 2]; both ranges are supported, including exact zero and
 * negative gates.  The readout after the update is the reading this library
 * implements (the pages print no readout).
 *
 * Entry points:
 *   kda_chunk_fwd   -- chunkwise-parallel WY forward over whole sequences
 *                      (prefill), the chunk-WY form of the SFDA page ("El
 *                      Teorema de Chunk-WY Constructivo") with the decay-
 *                      absorbed triangular solve of the Gated DeltaNet-2 page
 *                      (section 3), chunk C = 64;
 *   kda_decode_step -- one recurrent token with the state updated in place
 *                      (constant-memory inference, "Complex KDA" summary,
 *                      section on practical implications);
 *   kda_chunk_bwd   -- the gradients of the chunk forward (training), declared
 *                      with its workspace query further down.
 * Variants further down: the two-pass forward with a caller workspace, packed
 * variable-length batches, multi-token decode, Gated DeltaNet-2 gates and SFDA
 * complex gates, each with its backward.
 *
 * Conventions shared by all entry points
 *   - Every pointer except `shape` is a DEVICE pointer on the current HIP
 *     device; the caller owns every buffer.  The library allocates nothing,
 *     except the two-pass workspace that kda_chunk_fwd takes from the
 *     stream-ordered pool (see there).
 *   - Layouts are dense, row-major, contiguous:
 *       q, k, alpha : [B, T, H, dk]      (decode: [B, H, dk])
 *       v           : [B, T, H, dv]      (decode: [B, H, dv])
 *       beta        : [B, T, H]          (decode: [B, H])
 *       o           : [B, T, H, dv]      (decode: [B, H, dv]), same dtype as q
 *       states      : [B, H, dk, dv] fp32 (row = key channel, column = value channel)
 *     q, k, v, alpha, beta and o share one dtype (kda_dtype).
 *   - Alignment: states must be 16-byte aligned; kda_chunk_fwd also needs
 *     16-byte aligned q, k, v, alpha and o (they move in 16-byte vectors).
 *     Every other pointer needs only the alignment of its element type.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  The library keeps no mutable global state apart from
 *     kda_chunk_fwd_noalloc's per-GPU scratch array (calls of that entry point
 *     that overlap in time on one GPU race); concurrent calls of the others on
 *     different streams with disjoint outputs and workspaces are safe.
 *   - Return value: KDA_OK (0), or a negative kda_status.  Argument errors are
 *     detected on the host before anything is launched; KDA_ERR_HIP reports a
 *     launch failure (hipGetLastError).  No C++ exception crosses the ABI.
 *   - Preconditions that are documented but not checked on the device:
 *     |alpha| <= 1, 0 <= beta <= 2, k L2-normalised (these make every
 *     transition non-expansive).  Nothing is normalised or scaled inside.
 *     Gates with |alpha| below the smallest normal fp32 (~1.2e-38) may act
 *     as exact zeros.
 */
#ifndef KDA_H
#define KDA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_BF16 = 0, /* q, k, v, alpha, beta, o are bfloat16; state fp32 */
    KDA_F32 = 1   /* q, k, v, alpha, beta, o are float32; state fp32 */
} kda_dtype;

typedef struct {
    int B;          /* batch size, >= 0 */
    int T;          /* sequence length, >= 0 (ignored by kda_decode_step) */
    int H;          /* heads, >= 1 */
    int dk;         /* key channels: 64 or 128 */
    int dv;         /* value channels: 64 or 128 */
    int chunk;      /* chunk length; 0 or 64 (the only supported value) */
    kda_dtype dtype;
} kda_shape;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* negative / zero sizes, or sizes overflow */
    KDA_ERR_DTYPE = -3,       /* unknown kda_dtype */
    KDA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    KDA_ERR_ALIAS = -5,       /* the output overlaps an input it must not alias */
    KDA_ERR_UNSUPPORTED = -6, /* valid but unsupported (dk/dv, chunk, dtype x dk) */
    KDA_ERR_HIP = -7,         /* the HIP runtime reported an error on launch */
    KDA_ERR_WORKSPACE = -8,   /* workspace smaller than kda_chunk_fwd_workspace_size() */
    KDA_ERR_SCRATCH = -9      /* kda_chunk_fwd_noalloc: the shape needs more workspace than
                                 KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

/*
 * Chunkwise WY forward over whole sequences.
 *   initial_state : [B, H, dk, dv] fp32, or NULL for a zero start state.
 *   o             : [B, T, H, dv] output, must not overlap any input.
 *   final_state   : [B, H, dk, dv] fp32, or NULL (not written).  It may be
 *                   the same pointer as initial_state (each (b, h) tile is
 *                   read before it is written); any other overlap with an
 *                   input is KDA_ERR_ALIAS.
 * Supported: dk in {64, 128}, dv in {64, 128}; KDA_F32 requires dk == dv == 64.
 * T need not be a multiple of 64 (the last chunk is masked); B*T == 0 only
 * copies initial_state to final_state (or zeroes it).
 * Path: one chunk (T <= 64) runs the single-pass kernel; more than one chunk runs the
 * two-pass forward of kda_chunk_fwd_ws on a workspace of kda_chunk_fwd_workspace_size()
 * bytes that this call takes from the device's stream-ordered memory pool
 * (hipMallocAsync on `stream`) and hands back in stream order after the second pass
 * (hipFreeAsync); a pool failure is KDA_ERR_HIP.  Callers that manage their own memory
 * pass a workspace to kda_chunk_fwd_ws; callers that cannot allocate at all use
 * kda_chunk_fwd_noalloc.
 */
int kda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta, const float* initial_state,
                  void* o, float* final_state, void* stream);

/*
 * Two-pass chunk forward.  Same operation, arguments and errors as kda_chunk_fwd,
 * plus a caller-owned device workspace:
 *   pass 1 computes, for every (b, h, chunk) in parallel, the chunk's WY record into
 *          the workspace: for bf16 inputs A (the decay-weighted causal q.k products) and
 *          (I + T)^-1 diag(beta) as a bf16 pair (value and rounding residual); for
 *          fp32 inputs also -W, Q o gamma, (K o rho)^T and the last row's gamma;
 *   pass 2 walks the chunks of each (b, h) in order and carries the fp32 state
 *          (for bf16 it re-reads q, k, alpha and rebuilds the gate-scaled operands
 *          itself).
 *          With few (b, h) chains over a long sequence (bf16, dk = 128, at most 32
 *          64-column tiles), each chain is split into 8 or more segments of at least 16 chunks
 *          that are walked in parallel: once from a zero state (end state B_g), once
 *          from the identity with v = 0 (the segment's transfer P_g), then the start
 *          states S_(g+1) = P_g S_g + B_g are scanned and every segment is walked from
 *          its own start state (the affine block transfer of the SFDA page,
 *          "Principales Contribuciones" item 3); the scratch for this follows the
 *          records in the workspace and is counted by kda_chunk_fwd_workspace_size.
 * This trades extra HBM traffic (each record is written once and read once) for
 * parallelism over chunks; on MI355X it is the faster forward whenever T > 64 (about
 * twice the single-pass kernel at d = 128, measured from 128 to 2,048 heads), and for
 * bf16 the more exact one: its state chain carries the state, the residuals and
 * (I + T)^-1 diag(beta) as bf16 pairs, which keeps the norm-preserving regime (alpha
 * in {-1, +1}, beta in {0, 2}) at about 4e-3 at T = 65,536; the single-pass kernel pairs
 * the state and Delta only (W = (I + T)^-1 diag(beta) (K o gamma) stays single bf16) and
 * reaches about 1.9e-2 there at T = 8,192, near the 2e-2 bar, more beyond.
 *   workspace       : device memory, 256-byte aligned, not overlapping any argument;
 *                     NULL selects the single-pass kernel.
 *   workspace_bytes : at least kda_chunk_fwd_workspace_size(shape), else
 *                     KDA_ERR_WORKSPACE.
 * The workspace contents on return are unspecified.
 */
size_t kda_chunk_fwd_workspace_size(const kda_shape* shape);  /* 0 if the shape is invalid */
int kda_chunk_fwd_ws(const kda_shape* shape, const void* q, const void* k, const void* v,
                     const void* alpha, const void* beta, const float* initial_state,
                     void* o, float* final_state, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * kda_chunk_fwd_ws without a workspace argument and without any device allocation, for
 * callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments and errors as
 * kda_chunk_fwd_ws; the workspace is a fixed array of KDA_NOALLOC_SCRATCH_BYTES in device
 * memory that each GPU the library runs on holds from load until the process ends.
 *   limit : kda_chunk_fwd_workspace_size(shape) > KDA_NOALLOC_SCRATCH_BYTES is rejected
 *           with KDA_ERR_SCRATCH before anything runs (64 MiB holds about 3,100 (b, h,
 *           chunk) records: B*H = 32 heads up to T = 6,144 at d = 128, for instance).
 *   races : every call on one GPU uses that GPU's one array, so calls that overlap in
 *           time on the same GPU (different streams or host threads) must not be made;
 *           calls in one stream order are safe.  The array needs no clearing: a call reads
 *           only what it wrote itself.
 * The first call on a device (with that device current) looks up the array's device
 * address with hipGetSymbolAddress; a failure there is KDA_ERR_HIP.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_chunk_fwd_noalloc(const kda_shape* shape, const void* q, const void* k, const void* v,
                          const void* alpha, const void* beta, const float* initial_state,
                          void* o, float* final_state, void* stream);

/*
 * The two passes of kda_chunk_fwd_ws as separate calls (same workspace rules).
 * A chunk's record depends only on q, k, alpha and beta: with the chunk's q, k and
 * alpha it fixes the chunk's exact affine block transfer (SFDA page, "Principales
 * Contribuciones" item 3) less the part that v and the state enter linearly, so one
 * set of records can be applied to several v / start-state pairs of the same shape.
 *   kda_chunk_records       : reads q, k, alpha, beta [layouts as kda_chunk_fwd];
 *                             writes the records of every (b, h, chunk).
 *   kda_chunk_apply_records : reads the records, q, k, alpha (the same tensors the
 *                             records were made from: the walk rebuilds Q o gamma,
 *                             K o gamma and K o rho from them), v and initial_state
 *                             (NULL = zero); writes o and final_state (NULL = not
 *                             written; may equal initial_state).  The workspace is only
 *                             read.
 * shape->dv is checked but does not change the records.  Errors as kda_chunk_fwd_ws;
 * a NULL workspace is KDA_ERR_NULL unless the shape needs none (B*T == 0).
 */
int kda_chunk_records(const kda_shape* shape, const void* q, const void* k, const void* alpha,
                      const void* beta, void* workspace, size_t workspace_bytes, void* stream);
int kda_chunk_apply_records(const kda_shape* shape, const void* q, const void* k, const void* alpha,
                            const void* workspace, size_t workspace_bytes, const void* v,
                            const float* initial_state, void* o, float* final_state, void* stream);

/*
 * Packed variable-length batch (two-pass forward): n_seqs sequences lie back to back
 * along T, sequence i at token rows [cu_seqlens[i], cu_seqlens[i + 1]).  Each sequence
 * is cut into its own chunks of 64 (no chunk straddles two sequences) and runs the
 * recurrence from its own start state, exactly as a separate kda_chunk_fwd call would.
 *   shape->B        : must be 1 (KDA_ERR_SHAPE otherwise); shape->T = total tokens
 *   cu_seqlens      : DEVICE int32 [n_seqs + 1], 4-byte aligned; offsets are read on
 *                     the device, clamped to [0, T] and made non-decreasing
 *                     (cu_seqlens[0] is taken as 0); token rows after the last offset
 *                     belong to no sequence and are not written in o
 *   initial_state   : [n_seqs, H, dk, dv] fp32 or NULL (zeros)
 *   final_state     : [n_seqs, H, dk, dv] fp32 or NULL; may equal initial_state
 *   workspace       : kda_chunk_fwd_varlen_workspace_size(shape, n_seqs) bytes, 256-byte
 *                     aligned (records of at most ceil(T/64) + n_seqs chunks per head
 *                     and the chunk table)
 * q, k, alpha [1, T, H, dk], v and o [1, T, H, dv], beta [1, T, H]; other rules and
 * errors as kda_chunk_fwd_ws.  kda_gdn2_chunk_fwd_varlen takes the Gated DeltaNet-2
 * gates (below) in place of beta.
 */
size_t kda_chunk_fwd_varlen_workspace_size(const kda_shape* shape, int n_seqs); /* 0 if invalid */
int kda_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                         const void* k, const void* v, const void* alpha, const void* beta,
                         const float* initial_state, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);
int kda_gdn2_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs,
                              const void* q, const void* k, const void* v, const void* alpha,
                              const void* erase_gate, const void* write_gate,
                              const float* initial_state, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated DeltaNet-2 ("Gated DeltaNet-2" summary, section 1): the scalar beta is split
 * into an erase gate b_t per key channel and a write gate w_t per value channel,
 *   S_t = (I - k_t (b_t o k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t o v_t)^T,
 *   o_t = S_t^T q_t        (o: elementwise product; b = w = beta gives KDA).
 * The forward is the two-pass chunk forward of kda_chunk_fwd_ws (same workspace
 * size, kda_chunk_fwd_workspace_size; a workspace is required), with
 *   erase_gate : [B, T, H, dk], values in [0, 1] (the range is not checked)
 *   write_gate : [B, T, H, dv], values in [0, 1]
 * in the dtype of q and 16-byte aligned; no beta.  Other arguments, layouts, alias
 * rules and errors as kda_chunk_fwd_ws (the gates are inputs: no output may overlap
 * them).  The decode step takes erase_gate [B, H, dk] and write_gate [B, H, dv]
 * (element alignment) in place of beta and is otherwise kda_decode_step.
 */
int kda_gdn2_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                       const void* alpha, const void* erase_gate, const void* write_gate,
                       const float* initial_state, void* o, float* final_state,
                       void* workspace, size_t workspace_bytes, void* stream);
int kda_gdn2_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                         const void* alpha, const void* erase_gate, const void* write_gate,
                         float* state, void* o, void* stream);

/*
 * SFDA with phase control ("Resumen Tecnico: Atencion Delta de Fourier Semidirecta
 * (SFDA)", section "Arquitectura Central"): the real decay becomes the complex diagonal
 * Lambda_t = diag(alpha_t o e^{i theta_t}), applied in real coordinates as 2 x 2
 * rotation-decay blocks on key-channel pairs:
 *   S_t = (I - beta_t k_t k_t^T) Lambda_t S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *   (Lambda S)[2p]   = Re(l_p) S[2p] - Im(l_p) S[2p+1],
 *   (Lambda S)[2p+1] = Im(l_p) S[2p] + Re(l_p) S[2p+1]      (every state column),
 * where l_p = alpha_p e^{i theta_p} is the gate of coordinate p.  The chunk forward is
 * the exact chunk-WY product form of the same page ("El Teorema de Chunk-WY
 * Constructivo"), run as the two-pass forward of kda_chunk_fwd_ws.
 *   lambda : [B, T, H, dk] in the dtype of q, 16-byte aligned: channel 2p holds Re(l_p),
 *            channel 2p+1 holds Im(l_p) (|l_p| <= 1 is the intended range; not checked).
 *            Zero phases (Im = 0) give KDA with the two channels of a pair sharing a decay.
 * Other arguments, layouts, alias rules and errors as kda_chunk_fwd_ws (a workspace of
 * kda_chunk_fwd_workspace_size bytes is required); bf16 only (KDA_ERR_UNSUPPORTED for
 * fp32).  The varlen form takes the arguments of kda_chunk_fwd_varlen (its workspace
 * size).  The decode step and the multi-token decode take lambda [B, H, dk] (resp.
 * [B, T, H, dk]) in place of alpha, bf16 or fp32, otherwise as kda_decode_step and
 * kda_decode_tokens.
 */
int kda_sfda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                       const void* lambda, const void* beta, const float* initial_state, void* o,
                       float* final_state, void* workspace, size_t workspace_bytes, void* stream);
int kda_sfda_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs,
                              const void* q, const void* k, const void* v, const void* lambda,
                              const void* beta, const float* initial_state, void* o,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              void* stream);
int kda_sfda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                         const void* lambda, const void* beta, float* state, void* o, void* stream);
int kda_sfda_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* lambda, const void* beta, float* state, void* o,
                           void* stream);

/*
 * Backward of the chunk forward (training): the gradients of
 *   L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * through the KDA / CKDA forward of kda_chunk_fwd, with respect to q, k, v, alpha, beta
 * and the start state, taken through the same chunk-WY form (SFDA page, "El Teorema de
 * Chunk-WY Constructivo"; Gated DeltaNet-2 page, section 3, whose gate-aware backward
 * item keeps the per-channel gates inside the gradients of the intra-chunk matrices).
 * The forward is recomputed inside (the call takes the forward's inputs, not its
 * outputs).  Arithmetic is fp32 throughout (inputs widened from their dtype); the gate
 * gradient is formed without dividing by a gate, so exact zero gates get their exact
 * gradient.
 *   q, k, alpha, v, beta, initial_state : as kda_chunk_fwd (initial_state NULL = zeros)
 *   d_o             : [B, T, H, dv], dtype of q: the gradient of L with respect to o
 *   d_final_state   : [B, H, dk, dv] fp32, or NULL for a zero gradient of S_T
 *   dq, dk, dalpha  : [B, T, H, dk] fp32 outputs
 *   dv              : [B, T, H, dv] fp32 output
 *   dbeta           : [B, T, H] fp32 output
 *   d_initial_state : [B, H, dk, dv] fp32 output, or NULL when not wanted
 *   workspace       : kda_chunk_bwd_workspace_size(shape) bytes of device memory,
 *                     256-byte aligned (about 466 KB per chunk of 64 tokens and head at
 *                     dk = dv = 128; up to 512 slots of 320 KB for the gradient pass; and,
 *                     for few (b, h) over long sequences, the scratch of the split walks:
 *                     each chain's state and adjoint walks run as 8 or more parallel
 *                     segments joined by their affine transfers); its contents on entry do
 *                     not matter.
 * Supported: dk, dv in {64, 128}, bf16 or fp32 inputs, chunk 0 or 64.  q, k, v, alpha,
 * d_o, the outputs and the states need 16-byte alignment, beta that of its element type
 * (KDA_ERR_ALIGN otherwise).  No output may
 * overlap an input, another output or the workspace (KDA_ERR_ALIAS); a NULL required
 * pointer is KDA_ERR_NULL (unless B*T*H == 0), a short workspace KDA_ERR_WORKSPACE.
 * T == 0 writes d_initial_state = d_final_state (or zeros).
 */
size_t kda_chunk_bwd_workspace_size(const kda_shape* shape);  /* 0 if the shape is invalid */
int kda_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta, const float* initial_state,
                  const void* d_o, const float* d_final_state, float* dq, float* dk,
                  float* dv, float* dalpha, float* dbeta, float* d_initial_state,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward of a packed variable-length batch (the forward of kda_chunk_fwd_varlen):
 * shape->B must be 1 and shape->T is the total token count; n_seqs sequences lie back to
 * back at the device offsets cu_seqlens[0..n_seqs] (int32, non-decreasing, cu[0] = 0,
 * cu[n_seqs] <= T; out-of-range offsets are clamped).  Each sequence is differentiated on
 * its own, from its own start state: initial_state, d_final_state and d_initial_state are
 * [n_seqs, H, dk, dv] fp32 (NULL as for kda_chunk_bwd).  Tokens past cu[n_seqs] get no
 * gradient written.  workspace: kda_chunk_bwd_varlen_workspace_size(shape, n_seqs) bytes,
 * 256-byte aligned.  Other arguments, layouts and errors as kda_chunk_bwd; no output may
 * overlap cu_seqlens (KDA_ERR_ALIAS); a NULL cu_seqlens is KDA_ERR_NULL, B != 1 or
 * n_seqs < 0 KDA_ERR_SHAPE.
 */
size_t kda_chunk_bwd_varlen_workspace_size(const kda_shape* shape, int n_seqs);  /* 0 if invalid */
int kda_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                         const void* k, const void* v, const void* alpha, const void* beta,
                         const float* initial_state, const void* d_o, const float* d_final_state,
                         float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Backward of the Gated DeltaNet-2 chunk forward (kda_gdn2_chunk_fwd): the gate-aware
 * backward of the GDN-2 page (section 3), which keeps the erase gate b_t (per key
 * channel, on the read) and the write gate w_t (per value channel, on the write) inside
 * the gradients of the intra-chunk matrices.  With e = b o k per chunk,
 * T = [sum_c e_ic k_jc r_ijc] (j < i), W = (I + T)^-1 (E o gamma), U = (I + T)^-1 (w o V).
 *   erase_gate [B, T, H, dk], write_gate [B, T, H, dv] : inputs, dtype of q, 16-byte aligned
 *   d_erase [B, T, H, dk], d_write [B, T, H, dv] : fp32 outputs in place of dbeta
 * Everything else (workspace size kda_chunk_bwd_workspace_size / ..._varlen_workspace_size,
 * layouts, alignment, alias rules, errors, the packed form) as kda_chunk_bwd and
 * kda_chunk_bwd_varlen.
 */
int kda_gdn2_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                       const void* alpha, const void* erase_gate, const void* write_gate,
                       const float* initial_state, const void* d_o, const float* d_final_state,
                       float* dq, float* dk, float* dv, float* dalpha, float* d_erase,
                       float* d_write, float* d_initial_state, void* workspace,
                       size_t workspace_bytes, void* stream);
int kda_gdn2_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs,
                              const void* q, const void* k, const void* v, const void* alpha,
                              const void* erase_gate, const void* write_gate,
                              const float* initial_state, const void* d_o,
                              const float* d_final_state, float* dq, float* dk, float* dv,
                              float* dalpha, float* d_erase, float* d_write,
                              float* d_initial_state, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Backward of the SFDA chunk forward (kda_sfda_chunk_fwd; SFDA page, "Arquitectura
 * Central": complex rotation-decay gates).  lambda holds the gate of key-channel pair p as
 * (Re, Im) in channels (2p, 2p+1), as for the forward; dlambda [B, T, H, dk] fp32 returns
 * dL/dRe in channel 2p and dL/dIm in channel 2p+1.  The chunk form is kda_chunk_bwd's with
 * complex gate products per pair (r_ij = prod of lambda_l, j < l <= i): Q o gamma becomes
 * q conj(gamma), K o gamma k conj(gamma), K o rho rho k, the chunk-end decay rotates the
 * state's row pairs, and the gate gradient is the conjugate of the exclusive-product sum of
 * kda_chunk_bwd in complex arithmetic (no division by a gate).  Both dtypes; every other
 * argument, the workspace (kda_chunk_bwd_workspace_size / ..._varlen_workspace_size),
 * layouts, alignment, alias rules and errors as kda_chunk_bwd and kda_chunk_bwd_varlen.
 */
int kda_sfda_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                       const void* lambda, const void* beta, const float* initial_state,
                       const void* d_o, const float* d_final_state, float* dq, float* dk,
                       float* dv, float* dlambda, float* dbeta, float* d_initial_state,
                       void* workspace, size_t workspace_bytes, void* stream);
int kda_sfda_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs,
                              const void* q, const void* k, const void* v, const void* lambda,
                              const void* beta, const float* initial_state, const void* d_o,
                              const float* d_final_state, float* dq, float* dk, float* dv,
                              float* dlambda, float* dbeta, float* d_initial_state,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for every (b, h), state updated in place:
 *   S <- (I - beta k k^T) Diag(alpha) S + beta k v^T ;  o <- S^T q.
 *   state : [B, H, dk, dv] fp32, read and written in place.
 *   o     : [B, H, dv], must not overlap any input or the state.
 * shape->T and shape->chunk are ignored.  Supported: dk, dv in {64, 128}.
 */
int kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                    const void* alpha, const void* beta, float* state, void* o,
                    void* stream);

/*
 * Several tokens per (b, h) in one call (speculative / multi-token decoding): the
 * recurrence applied to shape->T consecutive tokens with the state read once, kept
 * on chip and written back once.
 *   q, k, alpha : [B, T, H, dk]; v : [B, T, H, dv]; beta : [B, T, H] (GDN-2: erase_gate
 *   [B, T, H, dk], write_gate [B, T, H, dv]); o : [B, T, H, dv], token t's readout after
 *   token t's update; state : [B, H, dk, dv] fp32, in place.
 * Same alignment, alias and error rules as kda_decode_step; T == 0 changes nothing.
 * The result equals T calls of kda_decode_step (up to fp32 summation order).
 */
int kda_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, float* state, void* o, void* stream);
int kda_gdn2_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* alpha, const void* erase_gate, const void* write_gate,
                           float* state, void* o, void* stream);

/* Human-readable text for a kda_status value (static storage). */
const char* kda_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int kda_version(void);

/*
 * Diagnostic: run the chunk forward like kda_chunk_fwd and also dump, for
 * every (b, h) and chunk, the chunk-local intermediates in fp32:
 *   dbg : [B*H, n_chunks, 4, 64, 64]  -> T (beta-scaled strictly lower),
 *                                        A (decay-weighted q.k, lower incl. diagonal),
 *                                        M = (I + T)^-1, and (I + T) M - I
 *                                        is not stored; slot 3 holds W[:, :64]
 * Used only by the test suite to localise a parity failure; slower than
 * kda_chunk_fwd.  Same arguments and errors as kda_chunk_fwd.
 */
int kda_chunk_fwd_debug(const kda_shape* shape, const void* q, const void* k, const void* v,
                        const void* alpha, const void* beta, const float* initial_state,
                        void* o, float* final_state, float* dbg, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
