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
  KDA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required */
  KDA_ERR_HIP = 6           /* the HIP runtime reported an error at launch */
} kda_status;

/* Entry points return their status as an int (one of kda_status) and take
 * the stream as void* (a hipStream_t), so the header needs no HIP include. */

/* Human-readable name of a status code (static storage). */
const char* kda_status_string(int status);

/* Build identity: a hex digest of the sources and compile flags the
 * library was built from (static storage).  Lets a caller (and the test
 * suite) check that the loaded binary was compiled from a given source
 * tree. */
const char* kda_build_id(void);

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
 * Numeric domain of the prefill (every kda_chunk_prefill* entry point
 * and the states they carry).  The carry's matrix products take v and the
 * running [K,V] state as fp16 operands (11-bit significand, float32
 * accumulation), so every |v| and every |state| entry -- the initial state
 * and every state the recurrence reaches -- must stay below 2^14 = 16384.
 * (On the workloads this library is measured on -- v of unit scale, initial
 * states of 0.1 -- the reached states stay below 1 in magnitude; a test
 * runs initial states up to the bound.)  Values outside the domain are not
 * detected (that would need a device-to-host read): they can overflow to
 * inf/NaN in o and final_state.
 * The decode path (kda_decode) works on float32 states and has no such
 * bound.
 */

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
 * Partition.  The page's design weighs two ways to spread this work, and
 * both are built: the split form (kda_chunk_prefill_split: a chip-wide
 * kernel writes each chunk's local matrices to the workspace, a second
 * kernel carries the state through them) and the fused form
 * (kda_chunk_prefill_fused: one workgroup per sequence and value head, no
 * workspace traffic).  They give the same results bit for bit.  This entry
 * point runs the fused form when N * HV (sequences times value heads) is at
 * least 3/4 of the device's compute units (192 on MI355X) and the split
 * form otherwise; kda_chunk_prefill_partition reports the choice.  Measured
 * on MI355X: the fused form takes 0.74-0.93 of the split form's time from
 * 192 units up and 1.7-2x at 96 units.  The workspace is checked either
 * way, so the errors a call returns do not depend on the device.
 *
 * Split-form schedule.  With sequences of equal length (cu_seqlens NULL,
 * or a single packed sequence), 48 to CUs - 32 (sequence, value head)
 * units, at least 48 chunks per sequence (24 when twice the units exceed
 * the compute units) and the whole workspace
 * kda_chunk_prefill_workspace_size returns (slots plus ready flags), the
 * split form overlaps its two kernels: the chunk kernel covers the first
 * chunks of every unit on every compute unit, then the rest beside the carry, which
 * runs on a second stream of the library's own (one per device, made on
 * the first such call that is not under graph capture, and kept; it forks
 * from and joins the caller's stream, which must belong to the current
 * device, so the call's work stays ordered on that stream, also under HIP
 * graph capture; a call captured before any uncaptured one runs
 * sequentially) and waits for each slot it reads to be flagged as stored.
 * If the runtime runs the carry before the chunk launch it waits for (a
 * runtime that serialises kernels, for example), the carry gives up after
 * a bounded wait (about 1 ms) and a sequential carry launched after the
 * join redoes those units, so the results do not depend on the two running
 * at once.  Otherwise the kernels run one after
 * the other.  Both schedules give the same results bit for bit; measured on
 * MI355X at T = 8192 the overlap takes 0.82-0.95 of the time.  The overlap
 * needs the library's stream on a hardware queue of its own: HIP spreads
 * a process's streams over a few hardware queues (GPU_MAX_HW_QUEUES, 4 by
 * default), and where the library's stream shares the caller's queue the
 * carry runs after the chunk kernel (measured 1.14 ms at B=1, H=HV=96,
 * T=8192 against 0.81 ms sequential, with seven copies of the library's
 * streams in one process).  A caller with many streams can keep the
 * sequential schedule by passing a workspace without the flag room.
 *
 *   q, k           bf16 [B, T, H, K]   raw (unnormalised) queries and keys
 *   v              bf16 [B, T, HV, V]  magnitudes below 2^14
 *   g              fp32 [B, T, HV, K]  per-channel log decay (finite, <= 0)
 *   beta           bf16 [B, T, HV]
 *   initial_state  fp32 [N, HV, K, V]  or NULL (zeros); entries below 2^14
 *                  in magnitude (see "Numeric domain" above)
 *   cu_seqlens     int32 [N + 1] device array of packed sequence offsets, or
 *                  NULL.  When given, B must be 1 and the N = num_seqs
 *                  sequences [cu[n], cu[n+1]) of the T axis are independent,
 *                  each with its own state; offsets must be non-decreasing,
 *                  start at 0 and end at T (not checked on the host).
 *                  When NULL, N = B and every batch row is one sequence.
 *   num_seqs       N when cu_seqlens is given (>= 1); ignored otherwise
 *   o              bf16 [B, T, HV, V]  output
 *   final_state    fp32 [N, HV, K, V]  output, always written
 *   workspace      device scratch owned by the caller, of
 *                  workspace_bytes >= HV * KDA_PREFILL_SLOT_BYTES (one
 *                  chunk slot per value head; fewer returns
 *                  KDA_ERR_WORKSPACE).  The split form runs in windows of
 *                  as many chunk slots as it holds, so
 *                  kda_chunk_prefill_workspace_size(...) bytes (one window
 *                  and the ready flags) is the fastest and a smaller
 *                  workspace trades speed for memory; bytes beyond that
 *                  size are not used.  When
 *                  kda_chunk_prefill_partition reports the fused form, the
 *                  workspace is checked but not touched, so the minimum
 *                  suffices.  Its contents on entry do not matter.
 *                  Calls that share a workspace must not overlap.
 * Sizes: B, T, H, HV >= 1 (T == 0 is accepted, may pass NULL token tensors,
 * and only writes final_state), HV <= 65535, HV % H == 0, K == V == 128.
 * q, k, v, g, beta, o and the workspace must not alias.
 */
#define KDA_PREFILL_SLOT_BYTES 66048
int kda_chunk_prefill(const void* q, const void* k, const void* v,
                      const float* g, const void* beta,
                      const float* initial_state,
                      const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t HV,
                      int32_t K, int32_t V,
                      void* o, float* final_state,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_split -- kda_chunk_prefill in the split form whatever
 * the unit count (same arguments, workspace rules and results).  For
 * callers that want the workspace-backed form explicitly, and for
 * measuring the two forms side by side.
 */
int kda_chunk_prefill_split(const void* q, const void* k, const void* v,
                            const float* g, const void* beta,
                            const float* initial_state,
                            const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t B, int32_t T, int32_t H, int32_t HV,
                            int32_t K, int32_t V,
                            void* o, float* final_state,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_partition -- the form kda_chunk_prefill (and
 * kda_chunk_prefill_noalloc) runs for these sizes on the current device:
 * KDA_PARTITION_SPLIT or KDA_PARTITION_FUSED (num_seqs as for
 * kda_chunk_prefill_workspace_size).  Returns -KDA_ERR_SHAPE for B or
 * HV < 1 or HV > 65535.  Host query; enqueues nothing.  When the runtime reports no
 * current device it answers for 256 compute units (MI355X).
 */
#define KDA_PARTITION_SPLIT 0
#define KDA_PARTITION_FUSED 1
int kda_chunk_prefill_partition(int32_t B, int32_t HV, int32_t num_seqs);

/*
 * kda_chunk_prefill_workspace_size -- bytes of workspace with which
 * kda_chunk_prefill runs fastest for these sizes (num_seqs as for
 * kda_chunk_prefill; pass 0 when cu_seqlens is NULL).  Returns 0 for sizes
 * kda_chunk_prefill rejects.
 * It is one 66048-byte block per 64-token chunk slot and value head, for
 * one window of min(floor(B*T/64) + N + 1, floor(2^31 / (HV * 66048)))
 * slots (about 1 KB per token and value head, at most about 2 GiB): the
 * prefill runs window by window over the slots and reuses the workspace.
 * When one window holds every slot, the overlapped schedule's ready flags
 * and unit status words follow: 4 bytes per (slot + sequence) and value
 * head, rounded up to 256 bytes.
 */
size_t kda_chunk_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV,
                                        int32_t K, int32_t V, int32_t num_seqs);

/*
 * kda_prefill_overlap_wait_limit -- testing hook for the overlapped split
 * schedule: the number of polls (about 55 ns each) its carry makes for one
 * ready flag before it gives up and leaves the unit to the sequential carry
 * after the join (default 16384, about 0.9 ms).  0 makes every wait give up
 * at once, which forces that path; a negative value restores the default.
 * Applies to calls enqueued afterwards; returns the previous value.  Not
 * needed in normal use.
 */
int32_t kda_prefill_overlap_wait_limit(int32_t polls);

/*
 * kda_chunk_prefill_noalloc -- kda_chunk_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same operation, arguments
 * and results (bit for bit), minus the workspace arguments.  The workspace
 * is instead a static device array inside the library,
 * KDA_NOALLOC_WORKSPACE_BYTES (64 MiB) per GPU, held from the library's
 * first use on that GPU until the process ends, and the split form runs in
 * windows of as many chunk slots as it holds.  It picks the partition as
 * kda_chunk_prefill does (the fused form does not touch the array).  This
 * entry point allocates and frees nothing.
 *
 * Limit: any B, T and N; HV <= 1016 (one 66048-byte slot per value head
 * must fit).  More value heads return KDA_ERR_WORKSPACE and enqueue nothing.
 * Every call on a GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results.  The
 * array needs no clearing: each call writes every part it reads.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                              const float* g, const void* beta,
                              const float* initial_state,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t B, int32_t T, int32_t H, int32_t HV,
                              int32_t K, int32_t V,
                              void* o, float* final_state, void* stream);

/*
 * kda_chunk_prefill_fused -- the same operation as kda_chunk_prefill, in
 * the fused partition: one workgroup per (sequence, value head) walks that
 * sequence's chunks in order and keeps everything on chip -- the chunk-local
 * matrices of each chunk go straight from LDS into the carry, against a
 * float32 state held in registers -- so no workspace is read or written.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3", sections "Function and
 * tensor contract" and "Mathematical definition", exactly as
 * kda_chunk_prefill (same arguments minus the workspace; the same results
 * as the split form bit for bit: both use the same per-chunk
 * arithmetic, operand precisions and accumulation orders).  It runs
 * whatever the unit count; it parallelises over N * HV (sequence, value
 * head) units only, so below about 3/4 of the compute units it leaves part
 * of the chip idle (see "Partition" under kda_chunk_prefill).
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
 * Batch invariance: a row's output and new state are the same bits
 * whatever the batch it is decoded in.  (Two kernels serve different batch
 * sizes -- column quarters of each (row, head) while 4 * B * HV is at most
 * the device's compute units, whole (row, head) pairs above -- and both
 * take the same arithmetic in the same order.)
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
 * specialised to H = 12), K == V == 128.  Batch invariant as kda_decode
 * (the same two kernels, chosen the same way).
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

/* Output dtypes of kda_chunk_backward's token gradients. */
enum {
  KDA_GRAD_FLOAT32 = 0,      /* dq, dk, dv, dbeta as float32 */
  KDA_GRAD_INPUT_DTYPE = 1   /* dq, dk, dv, dbeta in their inputs' dtype, bf16
                                (the float32 value rounded to nearest-even) */
};

/*
 * kda_chunk_backward -- gradients of the chunked prefill.
 *
 * Defined on "KDA Chunk Prefill on Ascend A3": section "Function and tensor
 * contract" (the optional backward) and the closing paragraph of section
 * "Timing and required submission" (the loss sum(o * do) + sum(final_state
 * * dht); gradients for q, k, v, g, beta and initial_state in their
 * corresponding dtypes, none for an absent initial state), with the forward
 * of section "Mathematical definition" exactly as kda_chunk_prefill.  The
 * page gives no backward formulas.  This computes the exact gradients of
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
 *   grad_dtype       KDA_GRAD_INPUT_DTYPE: dq, dk, dv and dbeta are bf16,
 *                    the dtype of q, k, v and beta (the page's contract);
 *                    KDA_GRAD_FLOAT32: they are float32 (the values before
 *                    that rounding).  Any other value: KDA_ERR_UNSUPPORTED.
 * Outputs (always written unless stated; all 16-byte aligned except dbeta):
 *   dq, dk           [B, T, H, K]   bf16 or float32 per grad_dtype (summed
 *                    over the value heads that share a Q/K head)
 *   dv               [B, T, HV, V]  bf16 or float32 per grad_dtype
 *   dg               [B, T, HV, K]  float32 (the dtype of g)
 *   dbeta            [B, T, HV]     bf16 or float32 per grad_dtype
 *   d_initial_state  fp32 [N, HV, K, V], or NULL to skip it (the page
 *                    returns none for an absent initial state; when
 *                    initial_state is NULL and this is given, it is the
 *                    gradient with respect to a zero initial state).
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
                       void* dq, void* dk, void* dv, float* dg, void* dbeta,
                       float* d_initial_state, int32_t grad_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_backward_workspace_size -- bytes of workspace kda_chunk_backward
 * needs (num_seqs as for kda_chunk_prefill; 0 when cu_seqlens is NULL);
 * 0 for sizes it rejects.  About 9.5 KB per token and value head: one
 * 557,568-byte record per 64-token chunk slot (floor(B*T/64) + N + 1
 * slots per value head) plus 1 KB per token and value head for the
 * per-value-head q and k gradients before the GQA sum.
 */
size_t kda_chunk_backward_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV,
                                         int32_t K, int32_t V, int32_t num_seqs);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
