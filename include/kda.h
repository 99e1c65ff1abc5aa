/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * The operation is the KDA forward hot path specified on the page
 * "KDA Chunk Prefill on Ascend A3" (sections "Function and tensor contract"
 * and "Mathematical definition") and, for single-token decode, on the page
 * "flashinfer.kda_decode.packed_kda_decode" (section "Parameters"), plus
 * the prefill's optional backward (kda_chunk_backward).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; all work is enqueued
 *     on `stream` (a hipStream_t; NULL selects the null stream).
 *   - bf16 tensors are arrays of IEEE bfloat16 bit patterns (uint16).
 *   - Tensors are dense and row-major in the listed axis order (last axis
 *     contiguous).  Pointers must be 16-byte aligned.
 *   - Inputs are read-only; only the named outputs (and, for kda_decode,
 *     the addressed slots of the state pool) are written.
 *   - Host-side checks cover metadata only (null pointers, sizes,
 *     alignment).  A failed check returns a nonzero status and enqueues
 *     nothing.  Device values are not inspected on the host.
 *   - After enqueueing, a launch error reported by the HIP runtime is
 *     returned as KDA_ERR_HIP.
 *   - K and V must both be 128 (the head width the pages' core cases use).
 *   - Fixed numerics, not parameters: query scale K**-0.5 and L2 epsilon
 *     1e-6 inside the square root.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,         /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
  KDA_ERR_UNSUPPORTED = 3,  /* valid request this build does not support (K, V != 128) */
  KDA_ERR_ALIGN = 4,        /* a pointer or stride is not 16-byte aligned */
  KDA_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
  KDA_ERR_WORKSPACE = 6     /* workspace missing or smaller than required */
} kda_status;

/* Human-readable name of a status code (static storage). */
const char* kda_status_string(int status);

/*
 * kda_qk_l2norm -- bit-exact row L2 normalisation of q or k.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3", section "Mathematical
 * definition": per row x of length K, in float32,
 *     y = bf16( x / sqrt( sum(x*x) + 1e-6 ) ).
 * The sum is the exact sum of the float32 squares rounded once to float32
 * (an order-free reading of the page's float32 reduction); the square root
 * and the division are correctly rounded float32 operations; the quotient
 * is rounded to bfloat16, nearest-even.  The same routine is fused into
 * kda_chunk_prefill and kda_decode, so their normalised values are equal
 * to this export's bit for bit.
 *
 *   x     bf16 [rows, K]   input rows (any Q/K tensor viewed as rows)
 *   y     bf16 [rows, K]   output; may not alias x
 *   rows  >= 0 (0 enqueues nothing)
 *   K     must be 128
 */
int kda_qk_l2norm(const void* x, void* y, int64_t rows, int32_t K, void* stream);

/*
 * kda_chunk_prefill -- KDA chunked prefill forward.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3": section "Function and tensor
 * contract" (forward(q, k, v, g, beta, initial_state) -> (o, final_state),
 * HV % H == 0, value head h reads Q/K head h // (HV / H)) and section
 * "Mathematical definition" (Q/K L2 normalisation as kda_qk_l2norm, then
 * the per-channel gated delta rule, computed chunk by chunk: chunk-local
 * G, L, A = solve(I+L, diag(beta)), W, U, Qg, Kg and Aqk, then the carry
 * Vnew = U - W S, O = Qg S + Aqk Vnew, S = exp(G_last) S + Kg^T Vnew).
 * The last partial chunk of each sequence behaves as if zero-padded, as
 * the page's golden does; o is written only for real tokens.
 *
 *   q, k           bf16 [B, T, H, K]   raw (unnormalised) queries and keys
 *   v              bf16 [B, T, HV, V]  magnitudes below 2^14
 *   g              fp32 [B, T, HV, K]  per-channel log decay (finite, <= 0)
 *   beta           bf16 [B, T, HV]
 *   initial_state  fp32 [N, HV, K, V]  or NULL (zeros)
 *   cu_seqlens     int32 [N + 1] device array of packed sequence offsets, or
 *                  NULL.  When given, B must be 1 and the N = num_seqs
 *                  sequences [cu[n], cu[n+1]) of the T axis are independent,
 *                  each with its own state; offsets must be non-decreasing,
 *                  start at 0 and end at T (not checked on the host).
 *                  When NULL, N = B and every batch row is one sequence.
 *   num_seqs       N when cu_seqlens is given (>= 1); ignored otherwise
 *   o              bf16 [B, T, HV, V]  output
 *   final_state    fp32 [N, HV, K, V]  output, always written
 *   workspace      device scratch of at least
 *                  kda_chunk_prefill_workspace_size(...) bytes, owned by the
 *                  caller; its contents on entry do not matter and are
 *                  overwritten (the chunk-local matrices of every chunk).
 *                  Calls that share a workspace must not overlap.
 * Sizes: B, T, H, HV >= 1 (T == 0 is accepted, may pass NULL token tensors,
 * and only writes final_state), HV % H == 0, K == V == 128.  q, k, v, g,
 * beta, o and the workspace must not alias.
 */
int kda_chunk_prefill(const void* q, const void* k, const void* v,
                      const float* g, const void* beta,
                      const float* initial_state,
                      const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t HV,
                      int32_t K, int32_t V,
                      void* o, float* final_state,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_workspace_size -- bytes of workspace kda_chunk_prefill
 * needs for these sizes (num_seqs as for kda_chunk_prefill; pass 0 when
 * cu_seqlens is NULL).  Returns 0 for sizes kda_chunk_prefill rejects.
 * It is about 1 KB per token and value head: one 66048-byte block per
 * 64-token chunk slot, with floor(B*T/64) + N + 1 slots per value head.
 */
size_t kda_chunk_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV,
                                        int32_t K, int32_t V, int32_t num_seqs);

/*
 * kda_chunk_prefill_fused -- the same operation as kda_chunk_prefill, in
 * the fused partition: one workgroup per (sequence, value head) walks that
 * sequence's chunks in order and keeps everything on chip -- the chunk-local
 * matrices of each chunk go straight from LDS into the carry, against a
 * float32 state held in registers -- so no workspace is read or written.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3", sections "Function and
 * tensor contract" and "Mathematical definition", exactly as
 * kda_chunk_prefill (same arguments minus the workspace, same results up
 * to floating-point rounding: both use the same per-chunk arithmetic and
 * operand precisions).  The page's design discussion weighs the two
 * partitions; this export lets them be measured side by side.  It
 * parallelises over N * HV (sequence, value head) units only, so it fills
 * the chip only when N * HV is at least the number of compute units.
 * Measured on MI355X (256 compute units): 2.0x slower than
 * kda_chunk_prefill at 96 units (B=1, HV=96, T=8192), even at 512 units
 * (16 variable-length sequences, HV=32) and 1.3x faster at 1024 units
 * (B=16, HV=64, T=2048) -- it saves the workspace round trip once the
 * units alone fill the chip twice over.
 */
int kda_chunk_prefill_fused(const void* q, const void* k, const void* v,
                            const float* g, const void* beta,
                            const float* initial_state,
                            const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t B, int32_t T, int32_t H, int32_t HV,
                            int32_t K, int32_t V,
                            void* o, float* final_state, void* stream);

/*
 * kda_decode -- one recurrent KDA step per batch row against a bf16 state
 * pool, updated in place.
 *
 * Defined on "flashinfer.kda_decode.packed_kda_decode", section
 * "Parameters" (caller-owned bf16 pool [N, HV, K, V] with compact inner
 * dimensions and a free outer slot stride; int32 slot index per row; -1
 * marks an inactive row that produces zero output and neither reads nor
 * writes the pool; scale 1/sqrt(128) and L2 epsilon 1e-6), and on "KDA
 * Chunk Prefill on Ascend A3", section "Mathematical definition" (the
 * recurrent step and the Q/K normalisation, as kda_qk_l2norm):
 *     S  = exp(g)[:,None] * pool[idx, hv]        (bf16 widened to fp32)
 *     r  = v - k^T S
 *     S' = S + beta k r^T
 *     o  = K**-0.5 q^T S'                        (from the unrounded S')
 *     pool[idx, hv] = bf16(S')                   (nearest-even)
 *
 *   q, k           bf16 [B, H, K]     (one token per row)
 *   v              bf16 [B, HV, V]
 *   g              fp32 [B, HV, K]
 *   beta           bf16 [B, HV]
 *   state_pool     bf16, slot s at state_pool + s * slot_stride elements,
 *                  each slot [HV, K, V] compact; slot_stride >= HV*K*V and a
 *                  multiple of 8 elements
 *   num_slots      number of slots in the pool
 *   state_indices  int32 [B] device array; active indices must be unique.
 *                  Any index outside [0, num_slots) -- including -1 -- is an
 *                  inactive row: zero output, no pool access.
 *   o              bf16 [B, HV, V]  (the [B, 1, HV, V] output)
 * Sizes: B >= 0 (0 enqueues nothing), H, HV >= 1, HV % H == 0,
 * K == V == 128.  Rows with the same active index race (undefined result).
 */
int kda_decode(const void* q, const void* k, const void* v,
               const float* g, const void* beta,
               void* state_pool, int64_t slot_stride, int64_t num_slots,
               const int32_t* state_indices,
               int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
               void* o, void* stream);

/*
 * kda_packed_decode -- kda_decode from the serving-native packed inputs:
 * Q/K/V extraction, the gate transform and the beta sigmoid fused into the
 * same kernel.
 *
 * Defined on "flashinfer.kda_decode.packed_kda_decode" (its description
 * and section "Parameters"): one post-convolution packed bf16 row per batch
 * row, raw per-channel gate logits and raw beta logits, per-head A_log and
 * per-channel dt_bias, lower_bound = -5; the state pool, slot indices,
 * -1 rows and output as kda_decode.  Per batch row b and head h
 * (H == HV; value head h reads Q/K head h):
 *     q, k, v = the three [H, K] blocks of mixed_qkv[b], in that order
 *     g       = -5 * sigmoid(exp(A_log[h]) * (raw_gate[b, h, :] + dt_bias[h, :]))
 *     beta    = sigmoid(raw_beta[b, h])
 * then exactly the step of kda_decode (normalisation, decay, delta update,
 * output, bf16 write-back), all in float32.  The page names the gate
 * transform, its parameters and its lower bound but prints no formula; the
 * line above is this library's reading of it.
 *
 *   mixed_qkv      bf16, row b at mixed_qkv + b * qkv_row_stride elements,
 *                  each row [3, H, K] compact; qkv_row_stride >= 3*H*K and a
 *                  multiple of 8 (the padding is never read)
 *   raw_gate       bf16 [B, H*K]
 *   raw_beta       bf16 [B, H]
 *   A_log          fp32 [H]
 *   dt_bias        fp32 [H*K]
 *   state_pool, slot_stride, num_slots, state_indices   as kda_decode (HV = H)
 *   o              bf16 [B, H, V]  (the [B, 1, H, V] output)
 * Sizes: B >= 0 (0 enqueues nothing), H >= 1 (the page's operator is
 * specialised to H = 12), K == V == 128.
 */
int kda_packed_decode(const void* mixed_qkv, int64_t qkv_row_stride,
                      const void* raw_gate, const void* raw_beta,
                      const float* A_log, const float* dt_bias,
                      void* state_pool, int64_t slot_stride, int64_t num_slots,
                      const int32_t* state_indices,
                      int32_t B, int32_t H, int32_t K, int32_t V,
                      void* o, void* stream);

/*
 * kda_state_to_pool -- prefill-to-decode handoff: store each sequence's
 * float32 state into its slot of the bf16 decode pool.
 *
 * Joins the two halves of the path: "KDA Chunk Prefill on Ascend A3",
 * section "Function and tensor contract" (the fp32 final_state
 * [N, HV, K, V] that kda_chunk_prefill returns) and
 * "flashinfer.kda_decode.packed_kda_decode", section "Parameters" (the
 * bf16 pool [slots, HV, K, V] that kda_decode reads and updates, with an
 * int32 slot index per row).  The stored value is the state rounded once
 * to bfloat16, nearest-even -- the same rounding kda_decode applies when it
 * writes a slot back.  NaN stays NaN (quiet); infinities and subnormals
 * round like any other value.
 *
 *   state          fp32 [N, HV, K, V]  input, read-only (e.g. final_state)
 *   N              number of states (>= 0; 0 enqueues nothing)
 *   state_pool     bf16, slot s at state_pool + s * slot_stride elements,
 *                  each slot [HV, K, V] compact; slot_stride >= HV*K*V and a
 *                  multiple of 8 elements
 *   num_slots      number of slots in the pool
 *   state_indices  int32 [N] device array: state n goes to slot
 *                  state_indices[n].  An index outside [0, num_slots) --
 *                  including -1 -- skips that state (no pool access).
 *                  Active indices must be unique (duplicates race).
 * Only the addressed slots are written; every other slot is untouched.
 * K == V == 128.
 */
int kda_state_to_pool(const float* state, int32_t N, int32_t HV, int32_t K, int32_t V,
                      void* state_pool, int64_t slot_stride, int64_t num_slots,
                      const int32_t* state_indices, void* stream);

/*
 * kda_chunk_backward -- gradients of the chunked prefill.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3": section "Function and tensor
 * contract" (the optional backward: gradients with respect to q, k, v, g,
 * beta and initial_state) and section "Mathematical definition" (the
 * forward being differentiated, exactly as kda_chunk_prefill).  The page
 * gives no backward formulas.  This computes the exact gradients of
 *     sum(o * d_out) + sum(final_state * d_final_state)
 * through the forward's definition, with one reading: the bf16 rounding of
 * the normalised q and k passes gradients unchanged, so dq and dk are the
 * gradients of x / sqrt(sum(x*x) + 1e-6) at the given q and k.  Every step
 * runs in float32 (it recomputes the chunk-local matrices, the chunk-start
 * states and the reverse state-gradient carry; it does not use the
 * forward's workspace or outputs).
 *
 * Inputs are the forward's inputs, with the same meaning and layout
 * (q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, HV, K,
 * V as for kda_chunk_prefill), plus:
 *   d_out            bf16 [B, T, HV, V]  gradient of o
 *   d_final_state    fp32 [N, HV, K, V]  gradient of final_state, or NULL
 *                    (zero)
 * Outputs (float32, always written unless stated; all 16-byte aligned):
 *   dq, dk           [B, T, H, K]   (summed over the value heads that share
 *                    a Q/K head)
 *   dv               [B, T, HV, V]
 *   dg               [B, T, HV, K]
 *   dbeta            [B, T, HV]
 *   d_initial_state  [N, HV, K, V], or NULL to skip it.  When initial_state
 *                    is NULL it is the gradient with respect to a zero
 *                    initial state.
 *   workspace        device scratch of at least
 *                    kda_chunk_backward_workspace_size(...) bytes, owned by
 *                    the caller; contents on entry do not matter.  Calls
 *                    that share a workspace must not overlap.
 * Sizes and errors as kda_chunk_prefill (T == 0 writes only
 * d_initial_state, which then equals d_final_state).  Outputs must not
 * alias inputs or each other.
 */
int kda_chunk_backward(const void* q, const void* k, const void* v,
                       const float* g, const void* beta,
                       const float* initial_state,
                       const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t HV,
                       int32_t K, int32_t V,
                       const void* d_out, const float* d_final_state,
                       float* dq, float* dk, float* dv, float* dg, float* dbeta,
                       float* d_initial_state,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_backward_workspace_size -- bytes of workspace kda_chunk_backward
 * needs (num_seqs as for kda_chunk_prefill; 0 when cu_seqlens is NULL);
 * 0 for sizes it rejects.  About 10.2 KB per token and value head: one
 * 590,336-byte record per 64-token chunk slot (floor(B*T/64) + N + 1
 * slots per value head) plus 1 KB per token and value head for the
 * per-value-head q and k gradients before the GQA sum.
 */
size_t kda_chunk_backward_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV,
                                         int32_t K, int32_t V, int32_t num_seqs);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
