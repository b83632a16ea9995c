/*
 * gdn.h - C ABI of the MI355X (gfx950) gated delta rule library, libgdn.so.
 *
 * The operator, per sequence and head, with a matrix state S of shape [d_v, d_k]:
 *
 *     S_t = S_{t-1} . alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,     o_t = S_t q_t
 *
 * Sources: paper note "Gated Delta Networks: Improving Mamba2 with Delta Rule"
 * (phantomic12 inference-research), mechanism paragraph (the recurrence, the parallel
 * WY / UT-transform training algorithm, a fixed-size per-head state with no KV cache);
 * record "LIT-137" (anthology-of-the-sota), "Standing in the anthology" (the same
 * recurrence; the WY-based chunkwise algorithm extended to carry the gate); module page
 * "Gated DeltaNet" (ai-model-reference), "How It Works" and "Math Or Compute Schema"
 * (the gate decays the old memory before the delta write; the query reads the updated
 * memory).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers allocated and owned by the caller. The
 *    library allocates nothing and keeps no pointer after a call returns. Its only state is
 *    a per-device cache of occupancy figures (filled on first use, safely under concurrent
 *    first calls) and the device scratch array of gdn_chunk_fwd_noalloc; calls on distinct
 *    streams may run concurrently (except overlapping gdn_chunk_fwd_noalloc calls on one GPU).
 *  - Layouts are dense, row-major, with the feature dimension innermost:
 *      q, k [B, T, H, d_k]     v, o [B, T, H, d_v]     g, beta [B, T, H]
 *      states (h0, hT, decode state) [N, H, d_v, d_k] fp32 (d_k contiguous)
 *    The pages list the state as (heads, d_k, d_v); the product v k^T makes it d_v x d_k,
 *    which is the stored order here.
 *  - dtype: GDN_F32 (q, k, v fp32) or GDN_BF16 (q, k, v bfloat16); o_dtype: GDN_F32 or
 *    GDN_BF16 (bf16 o only with bf16 inputs). g, beta and all states are fp32 in every
 *    case. Products run on the matrix cores with fp32 accumulation; bf16 inputs are
 *    multiplied as fp16 (exact for bf16 values of magnitude 2^-14..65504), which also
 *    carries the fp32 intermediates that become operands at 11 significant bits. A bf16 o
 *    is the fp32 result rounded to nearest even.
 *  - g is log(alpha) and must be <= 0 (alpha in (0, 1]); beta is used as given. Neither is
 *    checked on the device. There is no query scale (o_t = S_t q_t exactly).
 *  - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and the call
 *    returns at once. The return code reports host-side argument checks, which all run
 *    before any HIP call, and the status of the call's own kernel launches (an error left
 *    pending by an earlier, unrelated HIP call is neither reported nor cleared); faults
 *    during execution surface at the caller's next synchronisation.
 *  - GDN_CHECK=1 in the environment (a debugging aid): every entry point that takes
 *    cu_seqlens first copies it to the host, which synchronises `stream`, and returns
 *    GDN_ERR_SHAPE unless 0 = cu[0] <= cu[1] <= ... <= cu[N] = T.
 *  - GDN_SEGMENT_CHUNKS=L in the environment (for tests and tuning) fixes the segment length
 *    of the long-chain split of the bf16 forward pass to L chunks; 0 turns the split off.
 *    Without it the split is chosen from the shape (see gdn_chunk_fwd_workspace_bytes). The
 *    setting must not change between a workspace size query and the call that uses it.
 *  - GDN_FUSED=0 or 1 in the environment (for tests and tuning) forces gdn_chunk_fwd's path for
 *    bf16 inputs with dk = dv = 128: 0 the two stages, 1 the one-kernel forward (see
 *    gdn_chunk_fwd). It also selects the split plan, so the same rule about size queries holds.
 *  - Alignment: q, k, v, o, h0, hT and the decode state 16 bytes; g, beta and cu_seqlens
 *    4 bytes; the workspace 256 bytes. A misaligned pointer gives GDN_ERR_ALIGN.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    GDN_ERR_DTYPE = -3,       /* unknown dtype code */
    GDN_ERR_ALIGN = -4,       /* a pointer is misaligned */
    GDN_ERR_UNSUPPORTED = -5, /* chunk size or head dimension not built */
    GDN_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = -7          /* a HIP launch reported an error */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Library version, as major*10000 + minor*100 + patch. */
int gdn_version(void);

/* Human-readable text for a gdn_status value (static storage, never NULL). */
const char *gdn_status_string(int status);

/*
 * Workspace size in bytes needed by gdn_chunk_fwd / gdn_chunk_prepare /
 * gdn_chunk_propagate for the given problem (0 when no chunk exists). Pure host
 * function. `varlen` != 0 means cu_seqlens will be passed (then B must be 1 and N is
 * the number of packed sequences); otherwise N must equal B. Returns 0 for arguments
 * that the chunk entry points would reject.
 *
 * Workspace contents (all regions 256-byte aligned, in this order; `nc` is an upper
 * bound on the number of chunks, ceil(T/64)*B without cu_seqlens and
 * floor((T + N*63)/64) with them):
 *   chunk_base  int32 [2N + 1]        first chunk index of each sequence, the total, then the
 *                                     sequences by decreasing chunk count (varlen only)
 *   gates       fp32  [nc, H, 128]    exp(gamma_r) for r < 64, then exp(gamma_last - gamma_r),
 *                                     gamma = in-chunk inclusive cumulative sum of g
 *   Mmat        op    [nc, H, 64, 64] T diag(beta), T = (I + A)^{-1} (UT transform)
 *   P           op    [nc, H, 64, 64] (Q K^T) * exp(gamma_r - gamma_i) * [i <= r]
 *   K16         fp16  [nc, H, 64, dk] the chunk's K rows          (bf16 inputs only)
 *   Q16         fp16  [nc, H, 64, dk] diag(exp(gamma)) Q          (bf16 inputs only)
 * with op = fp16 for bf16 inputs and fp32 for fp32 inputs; rows and columns past a chunk's
 * last token are zero and gamma stays constant there. fp32 operators are row-major. The fp16
 * ones (Mmat, P, K16, Q16: W = 64 or dk columns) are stored as the LDS images the propagate
 * kernel reads: each row is W/8 pieces of 8 values, the piece at position pos of row r holds
 * columns 32(pc>>2) + 4(pc&3) + {0..3, 16..19} with pc = pos ^ swz(r), where
 * swz(r) = (4(r&3) + ((r>>2)&3)) ^ (r&2) for W = 128 and (r>>1)&7 for W = 64.
 * where A = strict_lower(diag(beta) K K^T * exp(gamma_r - gamma_i)).
 *
 * Long chains, bf16 inputs: the state propagation runs one work-group per (sequence, head,
 * 64-column d_v tile), or per 32-column tile when N*H*(dv/64) < 256 <= N*H*(dv/32). When
 * neither fills the device (N*H*(dv/64) at most 128) and a sequence can span at least 32
 * chunks, it cuts every sequence into `ns` segments of `sl` chunks (about 256 / (N*H*dv/64)
 * segments, each at least 16 chunks; the longest possible sequence, ceil(T/64) chunks, sets the
 * count). The one-kernel forward (see gdn_chunk_fwd) runs one work-group per (sequence, head)
 * and aims at about 256 / (N*H) segments of at least 8 chunks instead (a sequence that can span
 * 16 chunks or more). All segments run at once, segment 0 from h0 and the others from zero, recording
 * their final states and (segments past the first) their states at segment offsets 1, 2, 4, ..
 * below sl (`ncp` of them). A second pass reruns every segment at once from the final state
 * the first pass left for the segment before it, and stops at the first recorded offset where
 * its state equals the record bit for bit; a third walks the segments in order, accepts the
 * reruns whose starting state was the true one (every earlier segment matched) and recomputes
 * the rest from the true state. o and hT are bitwise those of the unsplit pass. The workspace
 * then ends with one more region:
 *   states      fp32  [N, H, ns, ncp + 2, dv, dk]   the recorded states, the first pass's final
 *                                                   state, the second pass's final state
 *                                                   (segments it did not match)
 *   reran       int32 [N, H, max(1, dv/64), ns]     chunks the second pass computed for each
 *                                                   segment s >= 1 of each 64-column tile
 *                                                   (a diagnostic; unset for segments past
 *                                                   the sequence's end)
 */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int varlen,
                                     int chunk, int dtype);

/*
 * Chunkwise-parallel forward pass (WY representation / UT transform carrying the
 * gate): computes o for every token and, optionally, the final state of every
 * sequence. Runs gdn_chunk_prepare followed by gdn_chunk_propagate on `stream` (bitwise the
 * same results), except for bf16 inputs with dk = dv = 128 and fewer than 64 (sequence, head)
 * pairs (or under GDN_FUSED=1): there one kernel builds each chunk's operators in LDS one chunk
 * ahead of the state propagation, reading q, k, v, g and beta once and writing only o, hT and
 * (long chains) the split's records. The two paths compute the same products in a different
 * order and agree to rounding; the stage-1 regions of the workspace are left untouched by the
 * one-kernel path.
 *
 *   q, k        [B, T, H, dk]  dtype                     (required)
 *   v           [B, T, H, dv]  dtype                     (required)
 *   g_log_alpha [B, T, H] fp32, log of the decay, <= 0   (required)
 *   beta        [B, T, H] fp32, write strength           (required)
 *   h0          [N, H, dv, dk] fp32 initial states, or NULL for zeros
 *   o           [B, T, H, dv]  o_dtype, written          (required)
 *   hT          [N, H, dv, dk] fp32 final states, written, or NULL. hT may be the same
 *               pointer as h0 (each state is read before it is overwritten); other
 *               overlaps are undefined.
 *   cu_seqlens  int32 [N + 1] device array of packed-sequence offsets, or NULL. With it,
 *               B must be 1 and sequence n covers tokens [cu[n], cu[n+1]) of the T axis;
 *               it must satisfy 0 = cu[0] <= cu[1] <= ... <= cu[N] = T (not checked on the
 *               device). Each sequence starts from h0[n] (or zeros); a zero-length one
 *               yields hT[n] = h0[n]. Without it, N must equal B and row b is sequence b.
 *   chunk       chunk length; 64 is the only one built
 *   B, T, H, dk, dv, N: sizes; dk, dv in {64, 128}; B, H >= 1; T >= 0; H <= 32768
 *   dtype       gdn_dtype of q, k and v
 *   o_dtype     gdn_dtype of o (GDN_F32, or GDN_BF16 when dtype is GDN_BF16)
 *   workspace   device scratch of at least gdn_chunk_fwd_workspace_bytes(...) bytes,
 *               owned by the caller; may be NULL only when that size is 0
 *   stream      hipStream_t to enqueue on
 * Returns GDN_OK or a negative gdn_status; nothing is launched on error.
 *
 * Value range, bf16 inputs: the state propagation multiplies fp16 operands (the state, K,
 * diag(e^gamma) Q, Mmat, P, the residual V - diag(e^gamma) K S^T and Delta = Mmat R) with fp32
 * accumulation. fp16 holds magnitudes up to 65504 and full relative precision down to 6.1e-5,
 * so the state entries, v and Delta must stay within about 3e4 in magnitude (beyond 65504 a
 * product operand becomes infinite and o turns non-finite), and values far below 1e-4 lose
 * relative precision. Within the tolerance of the workloads (2e-2 of the output RMS) the
 * kernels are tested at |v| up to 1.4e4, initial states of standard deviation 100, beta up to
 * 2, keys of length 1.4 (beta |k|^2 < 2: the recurrence contracts) and |v|, |h0| near 1e-3.
 * fp32 inputs use fp32 operands throughout.
 */
int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g_log_alpha,
                  const float *beta, const float *h0, void *o, float *hT,
                  const int32_t *cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                  int N, int dtype, int o_dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, arguments and
 * checks as gdn_chunk_fwd without the workspace arguments. Its kernels use, as their workspace,
 * a device array inside the library of GDN_NOALLOC_SCRATCH_BYTES bytes, of which every GPU the
 * library runs on holds its own copy until the process ends. The call allocates nothing.
 * A problem whose gdn_chunk_fwd_workspace_bytes(...) exceeds GDN_NOALLOC_SCRATCH_BYTES returns
 * GDN_ERR_WORKSPACE. Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels write every workspace byte they read, so nothing needs clearing):
 * calls that overlap in time on one GPU (different streams, or different host threads) race
 * and must not be issued.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g_log_alpha,
                          const float *beta, const float *h0, void *o, float *hT,
                          const int32_t *cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                          int N, int dtype, int o_dtype, void *stream);

/*
 * Stage 1 of gdn_chunk_fwd, independent across chunks (no state dependency): per
 * (chunk, head) the in-chunk gate scan and gate tables, the gated Gram matrix A, the UT
 * transform T = (I + A)^{-1} and the two chunk-local operators Mmat and P described above,
 * written to the workspace. Arguments as in gdn_chunk_fwd; v, h0, o and hT are not
 * used. Source: the WY / UT-transform chunkwise algorithm carrying the gate (paper note,
 * mechanism paragraph; record "LIT-137", "Standing in the anthology").
 */
int gdn_chunk_prepare(const void *q, const void *k, const float *g_log_alpha, const float *beta,
                      const int32_t *cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                      int N, int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stage 2 of gdn_chunk_fwd: for every (sequence, head) the state is carried through
 * the chunks in order, and each chunk's output is formed from the entering state and
 * the stage-1 operators:
 *     R = V - diag(e^gamma) K S^T,   Delta = Mmat R,   o = diag(e^gamma) Q S^T + P Delta,
 *     S <- e^{gamma_last} S + Delta^T diag(e^{gamma_last - gamma}) K.
 * Reads the workspace written by gdn_chunk_prepare with the same arguments on the same
 * stream. Arguments as in gdn_chunk_fwd; g_log_alpha and beta are not used.
 */
int gdn_chunk_propagate(const void *q, const void *k, const void *v, const float *h0, void *o,
                        float *hT, const int32_t *cu_seqlens, int chunk, int B, int T, int H,
                        int dk, int dv, int N, int dtype, int o_dtype, const void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Workspace size in bytes needed by gdn_chunk_bwd (arguments as in
 * gdn_chunk_fwd_workspace_bytes; 0 for arguments gdn_chunk_bwd would reject or when no
 * chunk exists). Contents, 256-byte aligned regions in this order (nc as above):
 *   the regions of gdn_chunk_fwd_workspace_bytes for fp32 operators (chunk_base, gates,
 *   Mmat, P; row-major [nc, H, 64, 64]; for bf16 inputs the Mmat region holds instead the
 *   fp16 LDS images of Mmat [nc, H, 64, 64] and then of P, as gdn_chunk_fwd's workspace
 *   stores them, and the P region the image of P - fp16(P) in fp16), then
 *   T        fp32 [nc, H, 64, 64]  (I + A)^{-1}, row-major (bf16 inputs: fp16)
 *   states   fp32 [nc, H, dv, dk]  the state entering each chunk (bf16 inputs: fp16, the
 *                                  precision its products take, and half the size)
 *   dstates  fp32 [nc, H, dv, dk]  the gradient reaching the state after each chunk
 *   K, Q     fp16 [nc, H, 64, dk] each, the LDS images of K and diag(e^gamma) Q (bf16 only).
 */
size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int varlen,
                                     int chunk, int dtype);

/*
 * Backward pass of gdn_chunk_fwd: given the gradients of a scalar loss with respect to
 * the outputs (d_o) and the final states (dhT), writes its gradients with respect to
 * q, k, v, g_log_alpha, beta and h0. The pages train the layer with the chunkwise
 * algorithm (paper note, mechanism paragraph: "parallel training algorithm") but print
 * no gradient formulas; these are the adjoint of the chunk equations of gdn_chunk_propagate,
 * computed chunk by chunk: stage 1 and 2 of the forward pass again (keeping T and the state
 * entering every chunk), a reverse walk over the chunks of each sequence carrying the
 * state gradient, then every (chunk, head) independently. fp32 inputs: all arithmetic is
 * fp32. bf16 inputs: the products run on fp16 operands with fp32 accumulation, fp32 states
 * and state gradients (the forward pass's numerics; the state entering each chunk is kept
 * for the per-chunk gradients in fp16, which is what their products take); the operands whose
 * rounding would dominate the per-chunk gradients are carried as fp16 hi + lo pairs. bf16 gradients are the
 * fp32 results rounded to nearest even.
 *
 *   q, k, v, g_log_alpha, beta, h0, cu_seqlens, chunk, B, T, H, dk, dv, N, dtype:
 *               the forward pass's arguments, as in gdn_chunk_fwd
 *   d_o         [B, T, H, dv] dtype, gradient with respect to o        (required)
 *   dhT         [N, H, dv, dk] fp32, gradient with respect to hT, or NULL for zeros
 *   dq, dk_out  [B, T, H, dk] grad_dtype, written                       (required)
 *   dv_out      [B, T, H, dv] grad_dtype, written                       (required)
 *   dg, dbeta   [B, T, H] fp32, written                                 (required)
 *   dh0         [N, H, dv, dk] fp32, written, or NULL (not written). Defined also when
 *               h0 is NULL (the gradient with respect to a zero initial state).
 *   grad_dtype  gdn_dtype of dq, dk_out, dv_out (GDN_F32, or GDN_BF16 when dtype is GDN_BF16)
 *   workspace   device scratch of at least gdn_chunk_bwd_workspace_bytes(...) bytes
 *   stream      hipStream_t to enqueue on
 * Outputs must not overlap inputs. Returns GDN_OK or a negative gdn_status; nothing is
 * launched on error.
 */
int gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g_log_alpha,
                  const float *beta, const float *h0, const void *d_o, const float *dhT,
                  void *dq, void *dk_out, void *dv_out, float *dg, float *dbeta, float *dh0,
                  const int32_t *cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                  int N, int dtype, int grad_dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * One recurrent decode step: one new token for each of N sequences and H heads,
 * applied to the states in place, with the readout of the updated state
 * (the recurrence above for a single t; the state is the whole memory, so decode
 * memory does not grow with context - paper note, mechanism paragraph).
 *
 *   q, k   [N, H, dk] dtype        v [N, H, dv] dtype
 *   g_log_alpha, beta  [N, H] fp32
 *   state  [N, H, dv, dk] fp32, read and overwritten in place
 *   o      [N, H, dv] in o_dtype (GDN_F32 or GDN_BF16), written. All arithmetic is
 *          fp32; a bf16 o is the fp32 result rounded to nearest even.
 * dk, dv in {64, 128}; N, H >= 1. Returns GDN_OK or a negative gdn_status.
 */
int gdn_decode_step(const void *q, const void *k, const void *v, const float *g_log_alpha,
                    const float *beta, float *state, void *o, int N, int H, int dk, int dv,
                    int dtype, int o_dtype, void *stream);

/*
 * Channel-wise decay (one decay per key channel): the pages extend the gated delta rule
 * "with a channel-wise forgetting gate" (record "LIT-137", "Standing in the anthology";
 * practice "SOTA-135", "Sequence") without a formula. The operator read from them:
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t,
 * alpha_t = exp(g_t) in (0,1]^{dk} scaling the state's key channels (its columns). With
 * the same g in every channel it is the operator of gdn_chunk_fwd.
 *
 * gdn_kda_chunk_fwd: chunkwise forward pass, arguments as in gdn_chunk_fwd except
 *   g_log_alpha [B, T, H, dk] fp32 (16-byte aligned), log of the per-channel decay, <= 0
 *   workspace   at least gdn_kda_chunk_fwd_workspace_bytes(...) bytes: chunk_base (packed
 *               only; as in gdn_chunk_fwd's workspace), then op [nc, H, 64, 64] Mmat and P, op [nc, H, 64, dk] K * e^gamma,
 *               Q * e^gamma and K * e^{gamma_last - gamma}, fp32 [nc, H, dk] e^{gamma_last}
 *               (gamma: per-channel in-chunk cumulative sum of g), with op = fp32 for fp32
 *               inputs and fp16 for bf16 inputs; row-major, except that for bf16 inputs the
 *               op arrays are stored as the LDS images of gdn_chunk_fwd's workspace.
 * Stage 1 computes in fp32 (bf16 inputs widened on load), except that for bf16 inputs the
 * products below the 16x16 diagonal blocks of A and P take fp16 operands (every gate factor
 * there is at most 1) and those of the diagonal blocks bf16 hi + lo operand pairs (three
 * products, about 16 significant bits per factor), with fp32 accumulation. Stage 2 multiplies fp32 operators
 * on the fp32 matrix core, and for bf16 inputs fp16 operators (the state packed to fp16 as
 * an operand, fp32 accumulation), as gdn_chunk_fwd does; a bf16 o is the fp32 result rounded
 * to nearest even.
 */
size_t gdn_kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int varlen,
                                         int chunk, int dtype);
int gdn_kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g_log_alpha,
                      const float *beta, const float *h0, void *o, float *hT,
                      const int32_t *cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                      int N, int dtype, int o_dtype, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * One decode step of the channel-wise-decay operator, arguments as in gdn_decode_step except
 * g_log_alpha [N, H, dk] fp32 (16-byte aligned). Per state row s_i: s~ = s_i * alpha,
 * c_i = beta (v_i - s~ . k), s_i <- s~ + c_i k, o_i = s~ . q + c_i (k . q).
 */
int gdn_kda_decode_step(const void *q, const void *k, const void *v, const float *g_log_alpha,
                        const float *beta, float *state, void *o, int N, int H, int dk, int dv,
                        int dtype, int o_dtype, void *stream);

/*
 * Decoupled channel-wise erase and write gates on top of the channel-wise decay: the pages
 * split beta "into a channel-wise erase gate and a channel-wise write gate on top of KDA's
 * channel-wise decay" (record "LIT-137", "Standing in the anthology"), the erase gate "on
 * the key", the write gate "on the value", with "the erased read" running "along a
 * reweighted key" (practice "SOTA-135", "Where it is incomplete"). The operator read from
 * them (tied scalar gates give the gated delta rule):
 *     Sa = S_{t-1} Diag(alpha_t),   S_t = Sa - (Sa (e_t * k_t)) k_t^T + (w_t * v_t) k_t^T,
 *     o_t = S_t q_t.
 * gdn_decoupled_chunk_fwd: as gdn_kda_chunk_fwd with beta replaced by
 *   erase [B, T, H, dk] fp32 and write [B, T, H, dv] fp32 (both required, 16-byte aligned);
 *   the workspace is the one of gdn_kda_chunk_fwd_workspace_bytes (Mmat holds T itself and
 *   the K * e^gamma region holds erase * K * e^gamma).
 * gdn_decoupled_decode_step: as gdn_kda_decode_step with erase [N, H, dk] and write
 *   [N, H, dv] in place of beta: c_i = w_i v_i - s~_i . (e * k), s_i <- s~_i + c_i k.
 */
int gdn_decoupled_chunk_fwd(const void *q, const void *k, const void *v, const float *g_log_alpha,
                            const float *erase, const float *write, const float *h0, void *o,
                            float *hT, const int32_t *cu_seqlens, int chunk, int B, int T, int H,
                            int dk, int dv, int N, int dtype, int o_dtype, void *workspace,
                            size_t workspace_bytes, void *stream);
int gdn_decoupled_decode_step(const void *q, const void *k, const void *v, const float *g_log_alpha,
                              const float *erase, const float *write, float *state, void *o, int N,
                              int H, int dk, int dv, int dtype, int o_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
